// Dense contractions of the step: the QKV, attention-output, MLP and tied
// vocabulary projections, forward and backward (Y = X W^T, dX = dY W,
// dW = dY^T X), with fused epilogues (bias, GELU with its derivative stored
// beside it for the backward, the product with that derivative, residual
// add). Matrix multiplication is where the time goes (Feste page, "Tensor
// Operations": matmul is the bottleneck); its CPU tiling for L1 is prior art,
// here the contraction runs on the gfx950 matrix cores.
//
// 16-bit path: bf16 or fp16 operands (E), v_mfma_f32_32x32x16_bf16 / _f16
// with fp32 accumulation:
//  * gemm16_kernel: block tile BM x BN (128 x 128, 4 wavefronts of 64 x 64,
//    two blocks per CU), K step 64, two LDS stages fed from registers loaded
//    two K steps ahead; LDS-staged epilogue.
//  * gemm16_pipe_kernel: persistent 256 x 256 tiles (8 wavefronts), direct
//    global-to-LDS loads in S stages, register epilogue; used where the
//    operand-load path rather than the matrix core bounds the 128 x 128 tile.
// Operands whose contiguous axis is M or N (the backward's dY^T and X^T, and W
// read along its rows for dX) stay in their memory layout in LDS and are read
// as MFMA fragments with the transposing LDS read.
//
// fp32 path: a plain LDS-tiled FMA kernel (64 x 64 tile, 4 x 4 per thread).
// Its vector-FMA peak is half the fp32 matrix-core peak (packed fp32
// instructions stay off in this build), but the fp32 workloads are a few
// hundred million flops per step and bound by launch latency, not by either.
#include <algorithm>
#include <cstdlib>
#include <cstring>
#include <type_traits>

#include "kernels.h"

namespace lm {

struct GemmArgs {
  const void* A;
  long lda;
  const void* B;
  long ldb;
  void* C;
  long ldc;
  const float* bias;
  const float* R;
  long ldr;
  void* aux;
  long ld_aux;
  int M, N, K;
  int M_out;          // rows < M_out are stored
  int k_split;        // K elements per blockIdx.z slice
  long split_stride;  // floats between the partial outputs of two slices
  float* colsum;      // GemmOp::colsum
};

// One GEMM of a grouped launch: its arguments, its first unit in the
// launch's unit numbering and its tile grid. The table ends with a sentinel
// entry whose first_unit is the launch's unit count.
struct GemmGroupEntry {
  GemmArgs a;
  int first_unit, tiles_m, tiles_n, pad;
};

// Epilogue of one output element (shared by both GEMM kernels and the
// split-K reduction). TA: activation storage type.
template <int EPI, typename TC, typename TA>
__device__ __forceinline__ void epilogue(const GemmArgs& p, long row, long col, float acc, int z) {
  if (EPI == EPI_PARTIAL) {
    reinterpret_cast<float*>(p.C)[z * p.split_stride + row * p.ldc + col] = acc;
  } else if (EPI == EPI_STORE) {
    float v = acc + (p.bias ? p.bias[col] : 0.f);
    Act<TC>::st(reinterpret_cast<TC*>(p.C), row * p.ldc + col, v);
  } else if (EPI == EPI_RESID) {
    float v = p.R[row * p.ldr + col] + acc + (p.bias ? p.bias[col] : 0.f);
    reinterpret_cast<float*>(p.C)[row * p.ldc + col] = v;
  } else if (EPI == EPI_GELU) {
    float g, d;
    gelu_and_grad(acc + (p.bias ? p.bias[col] : 0.f), g, d);
    Act<TA>::st(reinterpret_cast<TA*>(p.C), row * p.ldc + col, d);
    Act<TA>::st(reinterpret_cast<TA*>(p.aux), row * p.ld_aux + col, g);
  } else if (EPI == EPI_DGELU) {
    const float d = Act<TA>::ld(reinterpret_cast<const TA*>(p.aux), row * p.ld_aux + col);
    Act<TA>::st(reinterpret_cast<TA*>(p.C), row * p.ldc + col, acc * d);
  }
}

// Epilogue of 8 consecutive output columns (16-bit path; columns col..col+7
// exist, leading dimensions are multiples of 8).
template <typename E>
__device__ __forceinline__ void ld8_h(const void* p, float* v) {
  const uint4 u = *reinterpret_cast<const uint4*>(p);
  const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    v[2 * i] = H16<E>::lo(w[i]);
    v[2 * i + 1] = H16<E>::hi(w[i]);
  }
}
template <typename E>
__device__ __forceinline__ void st8_h(void* p, const float* v) {
  uint32_t w[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) w[i] = H16<E>::pack(v[2 * i], v[2 * i + 1]);
  *reinterpret_cast<uint4*>(p) = make_uint4(w[0], w[1], w[2], w[3]);
}
// 8 values as 16-bit through a buffer resource (an offset past the range is
// dropped; the store still counts as an outstanding memory operation)
typedef unsigned int w4_t __attribute__((ext_vector_type(4)));
template <typename E>
__device__ __forceinline__ void bst8_h(__amdgpu_buffer_rsrc_t r, unsigned off, const float* v) {
  w4_t w;
#pragma unroll
  for (int i = 0; i < 4; ++i) w[i] = H16<E>::pack(v[2 * i], v[2 * i + 1]);
  __builtin_amdgcn_raw_buffer_store_b128(w, r, (int)off, 0, 0);
}
__device__ __forceinline__ void ld8_f32(const float* p, float* v) {
  const float4 a = *reinterpret_cast<const float4*>(p), b = *reinterpret_cast<const float4*>(p + 4);
  v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w; v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
}
__device__ __forceinline__ void st8_f32(float* p, const float* v) {
  *reinterpret_cast<float4*>(p) = make_float4(v[0], v[1], v[2], v[3]);
  *reinterpret_cast<float4*>(p + 4) = make_float4(v[4], v[5], v[6], v[7]);
}

template <int EPI, typename TC, typename E>
__device__ __forceinline__ void epilogue8(const GemmArgs& p, long row, long col, float* v, int z) {
  if (EPI == EPI_PARTIAL) {
    st8_f32(reinterpret_cast<float*>(p.C) + z * p.split_stride + row * p.ldc + col, v);
    return;
  }
  if (EPI != EPI_DGELU && p.bias) {
    float b[8];
    ld8_f32(p.bias + col, b);
#pragma unroll
    for (int i = 0; i < 8; ++i) v[i] += b[i];
  }
  if (EPI == EPI_STORE) {
    if (sizeof(TC) == 4) st8_f32(reinterpret_cast<float*>(p.C) + row * p.ldc + col, v);
    else st8_h<E>(reinterpret_cast<E*>(p.C) + row * p.ldc + col, v);
  } else if (EPI == EPI_RESID) {
    float r[8];
    ld8_f32(p.R + row * p.ldr + col, r);
#pragma unroll
    for (int i = 0; i < 8; ++i) v[i] += r[i];
    st8_f32(reinterpret_cast<float*>(p.C) + row * p.ldc + col, v);
  } else if (EPI == EPI_GELU) {
    float a[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) gelu_and_grad(v[i], a[i], v[i]);
    st8_h<E>(reinterpret_cast<E*>(p.C) + row * p.ldc + col, v);
    st8_h<E>(reinterpret_cast<E*>(p.aux) + row * p.ld_aux + col, a);
  } else if (EPI == EPI_DGELU) {
    float d[8];
    ld8_h<E>(reinterpret_cast<const E*>(p.aux) + row * p.ld_aux + col, d);
#pragma unroll
    for (int i = 0; i < 8; ++i) v[i] *= d[i];
    st8_h<E>(reinterpret_cast<E*>(p.C) + row * p.ldc + col, v);
  }
}

// ---------------------------------------------------------- 16-bit MFMA GEMM
// Block tile BM x BN, K step 64, WGM x WGN wavefronts (wave tile WTM x WTN,
// multiples of 32), two LDS stages; global loads of step k+1 are issued before
// the MFMAs of step k.
//
// LDS layouts (no padding, XOR swizzles at 16-byte-chunk granularity):
//  K-contiguous operand: [row][64 k], 128 B per row; chunk c of row r sits at
//    c ^ ((r >> 1) & 7), so the 16-byte fragment reads of 16 consecutive rows
//    hit 64 distinct banks.
//  M/N-contiguous operand: [64 k][ROWS] copied as it is in memory (no register
//    transpose); chunk q of k-row k sits at q ^ ((k & 3) << 2). Its MFMA
//    fragments come from two ds_read_b64_tr_b16 per k-step: within each group
//    of 16 lanes, source lane i reads 4 elements at k-row k0 + i/4, columns
//    m0 + 4 (i % 4) .. + 3, and lane i receives column m0 + i at k-rows
//    k0 .. k0 + 3 (the layout of the instruction, checked on the device).
constexpr int kBK = 64;

template <int ROWS>
struct MNPitch {  // elements per k-row of an M/N-contiguous tile (>= 128 for the swizzle)
  static constexpr int value = ROWS < 128 ? 128 : ROWS;
};

typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) bf16x4_t lds_bf16x4;

// The LDS pointer is made by an address-space cast of the shared-array
// pointer (not through an integer), so the compiler keeps track of which LDS
// array a read comes from.
__device__ __forceinline__ bf16x4_t ds_read_tr(const bf16* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(const __attribute__((address_space(3))) bf16*)p);
}

typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));

template <int ROWS, bool KC, int NT>
struct Tile {
  static constexpr int PITCH = KC ? 64 : MNPitch<ROWS>::value;  // bf16 elements per LDS row
  static constexpr int ELEMS = KC ? ROWS * 64 : 64 * PITCH;
  static constexpr int CHUNKS = ROWS * 8;                        // 16-byte chunks per K step
  static constexpr int NL = (CHUNKS + NT - 1) / NT;
  static constexpr bool FULL = CHUNKS % NT == 0;                 // every thread owns NL chunks
  uint4 r[NL];
  __amdgpu_buffer_rsrc_t rsrc;
  unsigned voff[NL];  // byte offset of the chunk from the tile origin, without the K-step term
  int kin[NL];        // K offset of the chunk inside the K step
  int soff[NL];       // LDS element offset of the chunk
  bool cok[NL];       // the chunk's 8 columns exist (M/N-contiguous operand)
  unsigned kstride;   // bytes per unit of K

  // Per-thread addressing, computed once per block. The buffer starts at the
  // tile origin and ends after the operand's last element, so chunks outside
  // the operand read zeros (hardware range check) without a branch.
  __device__ __forceinline__ void init(const bf16* g, long ld, int row0, int rows_total, int K, int tid) {
    long origin, extent;
    if (KC) {
      origin = (long)row0 * ld;
      extent = (long)(rows_total - 1 - row0) * ld + K;
    } else {
      origin = row0;
      extent = (long)(K - 1) * ld + (rows_total - row0);
    }
    rsrc = __builtin_amdgcn_make_buffer_rsrc((void*)(g + origin), (short)0,
                                             (int)min(extent * 2, (long)0x7fffffff), 0x00020000);
    kstride = KC ? 2u : (unsigned)(ld * 2);
#pragma unroll
    for (int i = 0; i < NL; ++i) {
      const int c = min(tid + i * NT, CHUNKS - 1);
      if (KC) {
        const int row = c >> 3, kc = c & 7;
        voff[i] = (unsigned)(((long)row * ld + kc * 8) * 2);
        kin[i] = kc * 8;
        soff[i] = row * 64 + ((kc ^ ((row >> 1) & 7)) << 3);
      } else {
        const int k = c / (ROWS / 8), q = c % (ROWS / 8);
        voff[i] = (unsigned)(((long)k * ld + q * 8) * 2);
        kin[i] = k;
        soff[i] = k * PITCH + ((q ^ ((k & 3) << 2)) << 3);
      }
      cok[i] = KC || row0 + (c % (ROWS / 8)) * 8 < rows_total;
    }
  }

  // Loads of one K step (k0 .. k0 + 63, nothing at or past k_end) into rr.
  // The whole byte offset is in the per-lane offset, which the range check
  // covers.
  __device__ __forceinline__ void load(uint4* rr, int k0, int k_end) const {
    const unsigned ko = (unsigned)k0 * kstride;
#pragma unroll
    for (int i = 0; i < NL; ++i) {
      const unsigned vo = (cok[i] && k0 + kin[i] < k_end) ? voff[i] + ko : kOutOfRange;
      u32x4_t v = __builtin_amdgcn_raw_buffer_load_b128(rsrc, (int)vo, 0, 0);
      rr[i] = make_uint4(v[0], v[1], v[2], v[3]);
    }
  }
  __device__ __forceinline__ void load(int k0, int k_end) { load(r, k0, k_end); }

  __device__ __forceinline__ void store(const uint4* rr, bf16* __restrict__ s, int tid) const {
#pragma unroll
    for (int i = 0; i < NL; ++i)
      if (FULL || tid + i * NT < CHUNKS) *reinterpret_cast<uint4*>(s + soff[i]) = rr[i];
  }
  __device__ __forceinline__ void store(bf16* __restrict__ s, int tid) const { store(r, s, tid); }

  // MFMA 32x32x16 operand fragment: rows row0 + lane % 32, k-slots
  // ks*16 + 8 (lane / 32) .. + 7.
  __device__ __forceinline__ bf16x8_t frag(const bf16* __restrict__ s, int row0, int ks, int lane) const {
    if (KC) {
      const int row = row0 + (lane & 31);
      const int kc = ks * 2 + (lane >> 5);
      return *reinterpret_cast<const bf16x8_t*>(s + row * 64 + ((kc ^ ((row >> 1) & 7)) << 3));
    } else {
      const int g = lane >> 4, i = lane & 15;
      const int m = row0 + (g & 1) * 16 + 4 * (i & 3);  // first of the 4 columns this lane reads
      const int k = ks * 16 + (g >> 1) * 8 + (i >> 2);
      const int q = m >> 3, h = m & 7;
      const bf16* p0 = s + k * PITCH + (((q ^ ((k & 3) << 2))) << 3) + h;
      const bf16* p1 = s + (k + 4) * PITCH + (((q ^ (((k + 4) & 3) << 2))) << 3) + h;
      bf16x4_t lo = ds_read_tr(p0), hi = ds_read_tr(p1);
      return bf16x8_t{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    }
  }
};

// s_waitcnt with only the vector-memory counter limited to n (n < 64).

// Work unit u -> (tile m, tile n, K slice z). Units are numbered slice-major
// and, inside a slice, in groups of GM m-tiles walked n-tile by n-tile. Block
// b runs on XCD b % 8; the 32 blocks of one XCD take 32 consecutive units per
// round, so the panels they share stay in that XCD's L2.
__device__ __forceinline__ int pipe_unit(int round, int b, int nblocks) {
  const int xcd = b & 7, local = b >> 3;
  const int per_xcd = nblocks >> 3;  // nblocks is a multiple of 8
  return round * nblocks + xcd * per_xcd + local;
}
__device__ __forceinline__ void pipe_tile(int u, int tiles_m, int tiles_n, int& tm, int& tn, int& z) {
  const int tiles = tiles_m * tiles_n;
  z = u / tiles;
  const int t = u - z * tiles;
  constexpr int GM = 8;
  const int per_group = GM * tiles_n;
  const int group = t / per_group, first_m = group * GM;
  const int gsize = min(tiles_m - first_m, GM);
  const int in = t - group * per_group;
  tm = first_m + in % gsize;
  tn = in / gsize;
}

// Waves per SIMD of a configuration: blocks that fit the 160 KB LDS times the
// block's wavefronts, over the 4 SIMDs of a CU.
template <int BM, int BN, int WGM, int WGN>
struct GemmOcc {
  static constexpr int lds = 2 * 2 * (BM * 64 + BN * 64 + (BM < 128 ? 0 : 0));
  static constexpr int blocks = (160 * 1024) / lds > 0 ? (160 * 1024) / lds : 1;
  static constexpr int value = blocks * WGM * WGN / 4 > 0 ? blocks * WGM * WGN / 4 : 1;
};

// Persistent over work units (tile, K slice): the grid holds two blocks per
// CU and each block walks units with a stride of the grid (XCD-aware order,
// as for the 256 x 256 kernel). The first two K steps of a block's next unit
// are loaded into registers right after the current unit's K loop, so their
// latency hides behind the current unit's epilogue.
// k-step of the 128 x 128 kernel after whose MFMAs the next K step's
// registers are written to LDS (measured: after the third of four, 2-5%
// faster than after the last; after the second, slower).
constexpr int kStorePos = 2;
template <int BM, int BN, int WGM, int WGN, bool AK, bool BKC, int EPI, typename TC, typename E>
__global__ void __launch_bounds__(WGM * WGN * 64)
    __attribute__((amdgpu_waves_per_eu(GemmOcc<BM, BN, WGM, WGN>::value, GemmOcc<BM, BN, WGM, WGN>::value)))
    gemm16_kernel(GemmArgs p, int units) {
  constexpr int NT = WGM * WGN * 64;
  constexpr int WTM = BM / WGM, WTN = BN / WGN;
  constexpr int TM = WTM / 32, TN = WTN / 32;
  static_assert(TM * 32 == WTM && TN * 32 == WTN, "wave tiles are multiples of 32");
  using TA = Tile<BM, AK, NT>;
  using TB = Tile<BN, BKC, NT>;
  __shared__ __attribute__((aligned(16))) bf16 sA[2][TA::ELEMS];
  __shared__ __attribute__((aligned(16))) bf16 sB[2][TB::ELEMS];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave / WGN, wn = wave % WGN;
  const int tiles_m = (p.M + BM - 1) / BM, tiles_n = (p.N + BN - 1) / BN;
  const int nb = gridDim.x;
  const bf16* A = reinterpret_cast<const bf16*>(p.A);
  const bf16* B = reinterpret_cast<const bf16*>(p.B);
  // the K range of slice z
  auto k_range = [&](int z, int& kb, int& ke, int& nk) {
    kb = z * p.k_split;
    ke = min(p.K, kb + p.k_split);
    nk = (ke - kb + kBK - 1) / kBK;
  };

  TA la;
  TB lb;
  // Software pipeline, two K steps of global loads in flight: at step it the
  // LDS stage it%2 holds K step it, register set (it+1)%2 holds (or is
  // receiving) step it+1, and step it+2 is loaded into set it%2. Loads past
  // the last step re-load it (clamped) and are never read. Within a step the
  // fragments of k-step ks+1 are read while the MFMAs of ks run. The loop is
  // unrolled by two so the register sets stay static.
  uint4 ra[2][TA::NL], rb[2][TB::NL];
  bf16x8_t af[2][TM], bfr[2][TN];
  // set up the loaders for unit u and load its first two K steps
  auto prologue = [&](int u) {
    int tm, tn, z, kb, ke, nk;
    pipe_tile(u, tiles_m, tiles_n, tm, tn, z);
    k_range(z, kb, ke, nk);
    la.init(A, p.lda, tm * BM, p.M, p.K, tid);
    lb.init(B, p.ldb, tn * BN, p.N, p.K, tid);
    la.load(ra[0], kb, ke);
    lb.load(rb[0], kb, ke);
    la.load(ra[1], kb + min(1, max(nk - 1, 0)) * kBK, ke);
    lb.load(rb[1], kb + min(1, max(nk - 1, 0)) * kBK, ke);
  };

  // epilogue operands loaded ahead (one 8-column chunk per thread and pass):
  // GELU': this thread's chunks of the stored GELU'(u), at the unit's start, so their latency
  // hides behind the K loop; residual: the first wave row's fp32 chunks at
  // the unit's start, the next row's before each staging pass
  constexpr int CPT = WTM * BN / 8 / NT;  // epilogue chunks per thread and wave row
  constexpr bool PRE_U = EPI == EPI_DGELU && CPT * NT * 8 == WTM * BN;
  constexpr bool PRE_R = EPI == EPI_RESID && CPT * NT * 8 == WTM * BN;
  float4 rpre[PRE_R ? 2 * CPT : 1];
  uint4 upre[PRE_U ? WGM * CPT : 1];
  f32x16_t acc[TM][TN];
  constexpr int CP = BN + 4;
  static_assert(WTM * CP * 4 <= 2 * (TA::ELEMS + TB::ELEMS) * 2, "epilogue tile fits in the stage buffers");
  float* sC = reinterpret_cast<float*>(&sA[0][0]);

  // The next unit's first loads land while this unit's outputs are written;
  // epilogues that hold operands loaded ahead load a unit's first steps at
  // its start instead (the registers would not hold both).
  constexpr bool OVERLAP = !PRE_U && !PRE_R;
  int round = 0;
  int u = pipe_unit(0, blockIdx.x, nb);
  if (OVERLAP && u < units) prologue(u);
  for (; u < units; u = pipe_unit(++round, blockIdx.x, nb)) {
    if (!OVERLAP) prologue(u);
    int tm, tn, z, k_begin, k_end, nk;
    pipe_tile(u, tiles_m, tiles_n, tm, tn, z);
    k_range(z, k_begin, k_end, nk);
    const int m0 = tm * BM, n0 = tn * BN;
    // every thread issues its residual loads (outside the output: from the
    // residual's first element, the values then dropped), so the compiler
    // counts the loads in flight exactly and the stores need not wait for
    // one another
    auto load_r = [&](int w, int q, float4& lo, float4& hi) {
      const int c = tid + q * NT, r = c / (BN / 8), c8 = (c % (BN / 8)) * 8;
      const long row = m0 + w * WTM + r, col = n0 + c8;
      const bool ok = row < p.M_out && col < p.N;
      const float* src = p.R + (ok ? row * p.ldr + col : 0);
      lo = *reinterpret_cast<const float4*>(src);
      hi = *reinterpret_cast<const float4*>(src + 4);
      if (!ok) lo = hi = make_float4(0.f, 0.f, 0.f, 0.f);
    };
    if constexpr (PRE_R) {
#pragma unroll
      for (int q = 0; q < CPT; ++q) load_r(0, q, rpre[2 * q], rpre[2 * q + 1]);
    }
    if constexpr (PRE_U) {
#pragma unroll
      for (int w = 0; w < WGM; ++w)
#pragma unroll
        for (int q = 0; q < CPT; ++q) {
          const int c = tid + q * NT, r = c / (BN / 8), c8 = (c % (BN / 8)) * 8;
          const long row = m0 + w * WTM + r, col = n0 + c8;
          upre[w * CPT + q] =
              (row < p.M_out && col < p.N)
                  ? *reinterpret_cast<const uint4*>(reinterpret_cast<const E*>(p.aux) + row * p.ld_aux + col)
                  : make_uint4(0, 0, 0, 0);
        }
    }
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int j = 0; j < TN; ++j)
#pragma unroll
        for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;

    auto kstep = [&](int it) { return k_begin + min(it, max(nk - 1, 0)) * kBK; };
    la.store(ra[0], sA[0], tid);
    lb.store(rb[0], sB[0], tid);
    __syncthreads();

    auto step = [&](auto P_, int it) {
      constexpr int P = decltype(P_)::value;
      la.load(ra[P], kstep(it + 2), k_end);
      lb.load(rb[P], kstep(it + 2), k_end);
#pragma unroll
      for (int i = 0; i < TM; ++i) af[0][i] = la.frag(sA[P], wm * WTM + i * 32, 0, lane);
#pragma unroll
      for (int j = 0; j < TN; ++j) bfr[0][j] = lb.frag(sB[P], wn * WTN + j * 32, 0, lane);
#pragma unroll
      for (int ks = 0; ks < kBK / 16; ++ks) {
        const int f = ks & 1;
        if (ks + 1 < kBK / 16) {
#pragma unroll
          for (int i = 0; i < TM; ++i) af[f ^ 1][i] = la.frag(sA[P], wm * WTM + i * 32, ks + 1, lane);
#pragma unroll
          for (int j = 0; j < TN; ++j) bfr[f ^ 1][j] = lb.frag(sB[P], wn * WTN + j * 32, ks + 1, lane);
        }
        // keep the reads of k-step ks+1 ahead of the MFMAs of k-step ks
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int i = 0; i < TM; ++i)
#pragma unroll
          for (int j = 0; j < TN; ++j)
            acc[i][j] = mfma32<E>(af[f][i], bfr[f][j], acc[i][j]);
        // step it+1 into the other stage (free since the last barrier),
        // while the MFMAs of the remaining k-steps run
        if (ks == kStorePos) {
          la.store(ra[P ^ 1], sA[P ^ 1], tid);
          lb.store(rb[P ^ 1], sB[P ^ 1], tid);
        }
        __builtin_amdgcn_sched_barrier(0);
      }
      __syncthreads();
    };
    // Whole pairs in the loop and an odd last step after it: with no path
    // from the middle of a pair back to the loop head, the wait-count
    // analysis sees only the set being refilled as in flight at the head,
    // instead of waiting for every outstanding load there.
    int it = 0;
    for (; it + 1 < nk; it += 2) {
      step(std::integral_constant<int, 0>{}, it);
      step(std::integral_constant<int, 1>{}, it + 1);
    }
    if (it < nk) step(std::integral_constant<int, 0>{}, it);

    const int un = pipe_unit(round + 1, blockIdx.x, nb);
    if (OVERLAP && un < units) prologue(un);

    // Epilogue through LDS: the wave row w (WGN wavefronts, WTM rows) writes
    // its fp32 accumulators to LDS (row pitch BN + 4 floats), then all
    // threads walk that WTM x BN region in 8-column chunks, so bias, residual
    // and GELU operands are read and results written with 16- and 32-byte
    // accesses. Accumulator element e of tile (i, j): row (e/4)*8 +
    // (lane/32)*4 + e%4, column lane%32.
    auto stage_acc = [&](int w) {
      if (wm == w) {
#pragma unroll
        for (int i = 0; i < TM; ++i)
#pragma unroll
          for (int j = 0; j < TN; ++j)
#pragma unroll
            for (int e = 0; e < 16; ++e) {
              const int r = i * 32 + (e >> 2) * 8 + (lane >> 5) * 4 + (e & 3);
              const int c = wn * WTN + j * 32 + (lane & 31);
              sC[r * CP + c] = acc[i][j][e];
            }
      }
      __syncthreads();
    };
    if constexpr (PRE_U) {
#pragma unroll
      for (int w = 0; w < WGM; ++w) {
        stage_acc(w);
#pragma unroll
        for (int q = 0; q < CPT; ++q) {
          const int c = tid + q * NT, r = c / (BN / 8), c8 = (c % (BN / 8)) * 8;
          const long row = m0 + w * WTM + r, col = n0 + c8;
          if (row < p.M_out && col < p.N) {
            float v[8];
            ld8_f32(sC + r * CP + c8, v);
            const uint4 uu = upre[w * CPT + q];
            const uint32_t uw[4] = {uu.x, uu.y, uu.z, uu.w};
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              v[2 * i] *= H16<E>::lo(uw[i]);
              v[2 * i + 1] *= H16<E>::hi(uw[i]);
            }
            st8_h<E>(reinterpret_cast<E*>(p.C) + row * p.ldc + col, v);
          }
        }
        __syncthreads();
      }
    } else if constexpr (PRE_R) {
      // the bias of the thread's 8 columns, the same in every chunk, loaded
      // once: a load per chunk would wait for the stores before it (the
      // vector-memory counter retires in issue order)
      static_assert(NT % (BN / 8) == 0, "a thread's chunks share their columns");
      float bcol[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) bcol[i] = 0.f;
      {
        const long col = n0 + (tid % (BN / 8)) * 8;
        if (p.bias && col < p.N) ld8_f32(p.bias + col, bcol);
      }
#pragma unroll
      for (int w = 0; w < WGM; ++w) {
        float4 rnext[2 * CPT];
        if (w + 1 < WGM) {
#pragma unroll
          for (int q = 0; q < CPT; ++q) load_r(w + 1, q, rnext[2 * q], rnext[2 * q + 1]);
        }
        stage_acc(w);
#pragma unroll
        for (int q = 0; q < CPT; ++q) {
          const int c = tid + q * NT, r = c / (BN / 8), c8 = (c % (BN / 8)) * 8;
          const long row = m0 + w * WTM + r, col = n0 + c8;
          if (row < p.M_out && col < p.N) {
            float v[8];
            ld8_f32(sC + r * CP + c8, v);
#pragma unroll
            for (int i = 0; i < 8; ++i) v[i] += bcol[i];
            const float4 lo = rpre[2 * q], hi = rpre[2 * q + 1];
            v[0] += lo.x; v[1] += lo.y; v[2] += lo.z; v[3] += lo.w;
            v[4] += hi.x; v[5] += hi.y; v[6] += hi.z; v[7] += hi.w;
            st8_f32(reinterpret_cast<float*>(p.C) + row * p.ldc + col, v);
          }
        }
        if (w + 1 < WGM) {
#pragma unroll
          for (int q = 0; q < 2 * CPT; ++q) rpre[q] = rnext[q];
        }
        __syncthreads();
      }
    } else {
#pragma unroll 1
      for (int w = 0; w < WGM; ++w) {
        stage_acc(w);
        for (int c = tid; c < WTM * BN / 8; c += NT) {
          const int r = c / (BN / 8), c8 = (c % (BN / 8)) * 8;
          const long row = m0 + w * WTM + r, col = n0 + c8;
          if (row < p.M_out && col < p.N) {
            float v[8];
            ld8_f32(sC + r * CP + c8, v);
            epilogue8<EPI, TC, E>(p, row, col, v, z);
          }
        }
        __syncthreads();
      }
    }
  }
}

// --------------------------------------------------------------- fp32 GEMM
template <bool AK, bool BKC, int EPI>
__global__ void __launch_bounds__(256) gemm_f32_kernel(GemmArgs p) {
  constexpr int T = 64, KT = 16;
  __shared__ float sA[KT][T + 4];
  __shared__ float sB[KT][T + 4];
  const int tid = threadIdx.x, tx = tid & 15, ty = tid >> 4;
  const int m0 = blockIdx.y * T, n0 = blockIdx.x * T, z = blockIdx.z;
  const int k_begin = z * p.k_split, k_end = min(p.K, k_begin + p.k_split);
  const float* A = reinterpret_cast<const float*>(p.A);
  const float* B = reinterpret_cast<const float*>(p.B);
  float acc[4][4] = {};
  for (int k0 = k_begin; k0 < k_end; k0 += KT) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      int e = tid + q * 256;
      int row, k;
      if (AK) { row = e / KT; k = e % KT; } else { k = e / T; row = e % T; }
      int gr = m0 + row, gk = k0 + k;
      sA[k][row] = (gr < p.M && gk < k_end) ? (AK ? A[(long)gr * p.lda + gk] : A[(long)gk * p.lda + gr]) : 0.f;
      if (BKC) { row = e / KT; k = e % KT; } else { k = e / T; row = e % T; }
      gr = n0 + row;
      gk = k0 + k;
      sB[k][row] = (gr < p.N && gk < k_end) ? (BKC ? B[(long)gr * p.ldb + gk] : B[(long)gk * p.ldb + gr]) : 0.f;
    }
    __syncthreads();
#pragma unroll
    for (int k = 0; k < KT; ++k) {
      float a[4], b[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) a[i] = sA[k][ty + 16 * i];
#pragma unroll
      for (int j = 0; j < 4; ++j) b[j] = sB[k][tx + 16 * j];
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = fmaf(a[i], b[j], acc[i][j]);
    }
    __syncthreads();
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    long row = m0 + ty + 16 * i;
    if (row >= p.M_out) continue;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      long col = n0 + tx + 16 * j;
      if (col < p.N) epilogue<EPI, float, float>(p, row, col, acc[i][j], z);
    }
  }
}

// ---------------------------------------------------- split-K reduction
// Sums the S partial slices in slice order, then applies the real epilogue.
template <int EPI, typename TC, typename TA>
__global__ void splitk_reduce_kernel(GemmArgs p, const float* __restrict__ part, int S, long part_ld) {
  long idx = (long)blockIdx.x * blockDim.x + threadIdx.x;
  long total = (long)p.M_out * p.N;
  long stride = (long)gridDim.x * blockDim.x;
  for (; idx < total; idx += stride) {
    long row = idx / p.N, col = idx % p.N;
    float acc = 0.f;
    for (int z = 0; z < S; ++z) acc += part[(long)z * p.M * part_ld + row * part_ld + col];
    epilogue<EPI, TC, TA>(p, row, col, acc, 0);
  }
}

// --------------------------------------------- persistent pipelined GEMM
// Large tiles (256 x 256 with 8 wavefronts) cut the global-load bytes per
// flop to what one CU's load path sustains (about 50 B/clock measured, while
// a 128 x 128 tile needs 64 B/clock at the MFMA rate). Tiles arrive by
// direct-to-LDS loads in S stages of BK K-values; each stage is its own LDS
// array, so the compiler can tell that fragment reads of stage i do not
// depend on the loads still landing in the other stages, and the kernel
// itself waits (vmcnt) for exactly the loads of the step it is about to read.
//
// The MFMA takes the B fragment as its first operand, so a lane's
// accumulator holds one output row (lane % 32) and groups of 4 consecutive
// columns, which the epilogue writes straight from registers with 8- or
// 16-byte stores (no LDS staging, no barrier). Blocks are persistent: each
// walks work units (tile, K slice) with a stride of the grid, and the first
// loads of its next unit are issued before the epilogue of the current one.
//
// A direct load (buffer_load_dwordx4 ... lds) from lane j of a wavefront
// writes its 16 bytes at the wave's LDS base + 16 j (checked on the device),
// so each lane fetches the global chunk that belongs at its LDS slot under the
// swizzles below; no VGPR staging and no ds_write.

template <int ROWS, bool KC, int NT, int BK>
struct PTile {
  static_assert(ROWS == 128 || ROWS == 256 || ROWS == 192, "pipelined tiles hold 128, 192 or 256 rows");
  static_assert(BK == 32 || BK == 64, "K step of 32 or 64");
  static constexpr int CPR = BK / 8;                  // 16-byte chunks per K-contiguous row
  static constexpr int RPW = 128 / BK;                // K-contiguous rows per 256-byte bank window
  static constexpr int PITCH = KC ? BK : ROWS;        // bf16 elements per LDS row
  static constexpr int ELEMS = ROWS * BK;
  static constexpr int CHUNKS = ROWS * BK / 8;        // 16-byte chunks per K step
  static constexpr int NW = NT / 64;
  static constexpr int NI = CHUNKS / 64 / NW;         // load instructions per wavefront per K step
  static_assert(NI * 64 * NW == CHUNKS, "whole wavefront loads");
  __amdgpu_buffer_rsrc_t rsrc;
  unsigned voff[NI];
  int kin[NI];
  bool cok[NI];
  unsigned kstride;
  int wbase;

  // KC: chunk c of row r at position c ^ ((r / RPW) % CPR), so 16 lanes
  // reading 16 consecutive rows at one chunk cover distinct banks. MN: the
  // transposing reads of half a wavefront take 4 consecutive k-rows (k0 a
  // multiple of 4) x 4 chunks; chunk q of k-row k sits at q ^ mn_sw(k). With
  // a 256-byte-multiple row pitch (128 or 256 rows) every k-row starts on
  // bank 0 and mn_sw = (k & 3) << 2 puts the 4 rows on 4 distinct 16-bank
  // windows; with the 384-byte pitch of 192 rows, k-rows alternate between
  // banks 0 and 32, and mn_sw = ((k >> 1) & 1) << 2 separates the two rows
  // of each parity (the 4-chunk xor stays inside the row's 24 chunks).
  static __device__ __forceinline__ int kc_pos(int row, int c) { return c ^ ((row / RPW) % CPR); }
  static __device__ __forceinline__ int mn_sw(int k) { return ROWS == 192 ? ((k >> 1) & 1) << 2 : (k & 3) << 2; }

  __device__ __forceinline__ void setup(const bf16* g, long ld, int row0, int rows_total, int K, int tid) {
    long origin, extent;
    if (KC) {
      origin = (long)row0 * ld;
      extent = (long)(rows_total - 1 - row0) * ld + K;
    } else {
      origin = row0;
      extent = (long)(K - 1) * ld + (rows_total - row0);
    }
    rsrc = __builtin_amdgcn_make_buffer_rsrc((void*)(g + origin), (short)0,
                                             (int)min(extent * 2, (long)0x7fffffff), 0x00020000);
    kstride = KC ? 2u : (unsigned)(ld * 2);
    const int w = tid >> 6, lane = tid & 63;
    wbase = w * NI * 64;
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      const int pos = wbase + i * 64 + lane;  // LDS slot this lane fills
      if (KC) {
        const int row = pos / CPR, kc = kc_pos(row, pos % CPR);
        voff[i] = (unsigned)(((long)row * ld + kc * 8) * 2);
        kin[i] = kc * 8;
        cok[i] = true;
      } else {
        const int k = pos / (ROWS / 8), q = (pos % (ROWS / 8)) ^ mn_sw(k);
        voff[i] = (unsigned)(((long)k * ld + q * 8) * 2);
        kin[i] = k;
        cok[i] = row0 + q * 8 < rows_total;
      }
    }
  }

  // Issue the loads of the K step at k0 into the stage tile s (asynchronous).
  __device__ __forceinline__ void load(bf16* s, int k0, int k_end) const {
    const unsigned ko = (unsigned)k0 * kstride;
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      const unsigned vo = (cok[i] && k0 + kin[i] < k_end) ? voff[i] + ko : kOutOfRange;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (lds_void_t*)(s + (wbase + i * 64) * 8), 16, (int)vo, 0, 0, 0);
    }
  }

  // MFMA 32x32x16 operand fragment: rows row0 + lane % 32, k-slots
  // ks*16 + 8 (lane / 32) .. + 7.
  static __device__ __forceinline__ bf16x8_t frag(const bf16* __restrict__ s, int row0, int ks, int lane) {
    if (KC) {
      const int row = row0 + (lane & 31);
      const int kc = ks * 2 + (lane >> 5);
      return *reinterpret_cast<const bf16x8_t*>(s + row * BK + (kc_pos(row, kc) << 3));
    } else {
      const int g = lane >> 4, i = lane & 15;
      const int m = row0 + (g & 1) * 16 + 4 * (i & 3);
      const int k = ks * 16 + (g >> 1) * 8 + (i >> 2);
      const int q = m >> 3, h = m & 7;
      const bf16* p0 = s + k * PITCH + ((q ^ mn_sw(k)) << 3) + h;
      const bf16* p1 = s + (k + 4) * PITCH + ((q ^ mn_sw(k + 4)) << 3) + h;
      bf16x4_t lo = ds_read_tr(p0), hi = ds_read_tr(p1);
      return bf16x8_t{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    }
  }
};

// One LDS array per pipeline stage and operand (a distinct object per I).
template <int I, int ELEMS>
__device__ __forceinline__ bf16* lds_stage() {
  __shared__ __attribute__((aligned(1024))) bf16 buf[ELEMS];
  return buf;
}



// Epilogue of 4 consecutive output columns col..col+3 of one row.
template <int EPI, typename TC, typename E>
__device__ __forceinline__ void epilogue4(const GemmArgs& p, long row, long col, f32x4_t v, int z) {
  if (EPI == EPI_PARTIAL) {
    *reinterpret_cast<f32x4_t*>(reinterpret_cast<float*>(p.C) + z * p.split_stride + row * p.ldc + col) = v;
    return;
  }
  if (EPI != EPI_DGELU && p.bias) v += *reinterpret_cast<const f32x4_t*>(p.bias + col);
  auto st4 = [](E* d, f32x4_t x) {
    *reinterpret_cast<uint2*>(d) = make_uint2(H16<E>::pack(x[0], x[1]), H16<E>::pack(x[2], x[3]));
  };
  if (EPI == EPI_STORE) {
    if (sizeof(TC) == 4) *reinterpret_cast<f32x4_t*>(reinterpret_cast<float*>(p.C) + row * p.ldc + col) = v;
    else st4(reinterpret_cast<E*>(p.C) + row * p.ldc + col, v);
  } else if (EPI == EPI_RESID) {
    v += *reinterpret_cast<const f32x4_t*>(p.R + row * p.ldr + col);
    *reinterpret_cast<f32x4_t*>(reinterpret_cast<float*>(p.C) + row * p.ldc + col) = v;
  } else if (EPI == EPI_GELU) {
    f32x4_t a, d;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      float gi, di;
      gelu_and_grad(v[i], gi, di);
      a[i] = gi;
      d[i] = di;
    }
    st4(reinterpret_cast<E*>(p.C) + row * p.ldc + col, d);
    st4(reinterpret_cast<E*>(p.aux) + row * p.ld_aux + col, a);
  } else if (EPI == EPI_DGELU) {
    const uint2 u = *reinterpret_cast<const uint2*>(reinterpret_cast<const E*>(p.aux) + row * p.ld_aux + col);
    v[0] *= H16<E>::lo(u.x);
    v[1] *= H16<E>::hi(u.x);
    v[2] *= H16<E>::lo(u.y);
    v[3] *= H16<E>::hi(u.y);
    st4(reinterpret_cast<E*>(p.C) + row * p.ldc + col, v);
  }
}

// Split-K reduction, 4 columns per thread (N a multiple of 4, leading
// dimensions multiples of 8): sums the S partial slices in slice order, then
// applies the real epilogue.
template <int EPI, typename TC, typename E>
__global__ void __launch_bounds__(256) splitk_reduce4_kernel(GemmArgs p, const float* __restrict__ part, int S,
                                                            long part_ld) {
  const int nq = p.N >> 2;
  const long total = (long)p.M_out * nq;
  const long slice = (long)p.M * part_ld;
  for (long q = (long)blockIdx.x * blockDim.x + threadIdx.x; q < total; q += (long)gridDim.x * blockDim.x) {
    const long row = q / nq, col = (q - row * nq) * 4;
    // each partial is read once: nontemporal loads
    const f32x4_t* src = reinterpret_cast<const f32x4_t*>(part + row * part_ld + col);
    const long sl4 = slice / 4;
    f32x4_t acc = __builtin_nontemporal_load(src);
    int z = 1;
    for (; z + 3 < S; z += 4) {
      const f32x4_t a = __builtin_nontemporal_load(src + z * sl4);
      const f32x4_t b = __builtin_nontemporal_load(src + (z + 1) * sl4);
      const f32x4_t c = __builtin_nontemporal_load(src + (z + 2) * sl4);
      const f32x4_t d = __builtin_nontemporal_load(src + (z + 3) * sl4);
      acc += a;
      acc += b;
      acc += c;
      acc += d;
    }
    for (; z < S; ++z) acc += __builtin_nontemporal_load(src + z * sl4);
    epilogue4<EPI, TC, E>(p, row, col, acc, 0);
  }
}

template <int BM, int BN, int WGM, int WGN, int BK, int S, int OCC, bool AK, bool BKC, int EPI, typename TC,
          typename E>
__global__ void __launch_bounds__(WGM * WGN * 64) __attribute__((amdgpu_waves_per_eu(OCC, OCC)))
    gemm16_pipe_kernel(GemmArgs p, int units, int tiles_m, int tiles_n) {
  constexpr int NT = WGM * WGN * 64;
  constexpr int WTM = BM / WGM, WTN = BN / WGN;
  constexpr int TM = WTM / 32, TN = WTN / 32;
  static_assert(TM * 32 == WTM && TN * 32 == WTN, "wave tiles are multiples of 32");
  static_assert(S >= 2, "at least two stages");
  using LA = PTile<BM, AK, NT, BK>;
  using LB = PTile<BN, BKC, NT, BK>;
  constexpr int NLD = LA::NI + LB::NI;       // load instructions per wavefront per K step
  constexpr int KS = BK / 16;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave / WGN, wn = wave % WGN;
  const bf16* A = reinterpret_cast<const bf16*>(p.A);
  const bf16* B = reinterpret_cast<const bf16*>(p.B);
  const int nb = gridDim.x;

  LA la;
  LB lb;
  // A and B tiles of a stage are separate arrays: the compiler then keeps
  // the direct loads into one apart from the reads of the others.
  auto stage = [](auto I_) -> bf16* { return lds_stage<2 * decltype(I_)::value, LA::ELEMS>(); };
  auto stage_b = [](auto I_) -> bf16* { return lds_stage<2 * decltype(I_)::value + 1, LB::ELEMS>(); };
  auto k_range = [&](int z, int& kb, int& ke) {
    kb = z * p.k_split;
    ke = min(p.K, kb + p.k_split);
  };
  // Output chunks of a lane in epilogue pass i (accumulator rows i*32 ..
  // +31 of the wave tile): chunk q is row q*RPQ + lane / (64 / RPQ), columns
  // from (lane % (64 / RPQ)) * CW, CW = 8 for 16-bit outputs, 4 for fp32.
  constexpr bool H = sizeof(TC) == 2;
  constexpr int CW = H ? 8 : 4, LPR = 64 / CW, RPQ = 64 / LPR, NQ = 32 / RPQ;
  // The residual or the stored GELU'(u) is loaded ahead into registers (when
  // the wave tile is small enough to keep them): the passes i < PRE_I with the
  // unit's first K steps, so their latency hides behind the K loop, the others
  // at the start of the epilogue. (Two passes of the 16-bit GELU'(u) take 32
  // VGPRs, one pass of the fp32 residual as many.)
  constexpr bool PRE = (EPI == EPI_RESID || EPI == EPI_DGELU) && TM <= 2;
  // 16-bit plain and GELU outputs: the next unit's first loads are issued
  // before the outputs, which go out through buffer stores (an out-of-range
  // offset is dropped but still counted), so the next unit's first wait can
  // leave exactly NST stores of each wavefront in flight
  constexpr bool EARLY = ((EPI == EPI_STORE && TM <= 3) || (EPI == EPI_GELU && TM <= 2)) && H && S == 2 && !PRE;
  constexpr int PRE_I = EPI == EPI_DGELU ? TM : 1;
  uint4 pre[PRE ? TM : 1][PRE ? NQ : 1];
  // Through a buffer resource from the tile's origin: every lane issues its
  // load (an offset past the range reads zeros), so the number of loads in
  // flight after a unit's first K steps is known exactly.
  auto load_pre = [&](int tm, int tn, int i) {
    constexpr int ES = EPI == EPI_DGELU ? 2 : 4;  // 8 16-bit or 4 fp32 values
    const long r0 = (long)tm * BM, c0 = (long)tn * BN;
    const long ld = EPI == EPI_DGELU ? p.ld_aux : p.ldr;
    const char* base = EPI == EPI_DGELU ? reinterpret_cast<const char*>(p.aux) : reinterpret_cast<const char*>(p.R);
    const long n = r0 < p.M_out ? ((p.M_out - 1 - r0) * ld + p.N - c0) * ES : 0;
    const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(base + (r0 * ld + c0) * ES), (short)0, (int)min(n, (long)0x7fffffff), 0x00020000);
    // offsets within the tile fit in 32 bits (the dispatcher checks the
    // leading dimensions)
    const int ldi = (int)ld, rows = (int)min((long)BM, p.M_out - r0), cols = (int)min((long)BN, p.N - c0);
    const int lr0 = wm * WTM + i * 32 + lane / LPR, lc = wn * WTN + (lane % LPR) * CW;
#pragma unroll
    for (int q = 0; q < NQ; ++q) {
      const int lr = lr0 + q * RPQ;
      const bool ok = lr < rows && lc < cols;
      const w4_t w = __builtin_amdgcn_raw_buffer_load_b128(r, ok ? (lr * ldi + lc) * ES : (int)kOutOfRange, 0, 0);
      pre[i][q] = make_uint4(w[0], w[1], w[2], w[3]);
    }
  };
  // set up the loaders of unit u and issue its first S - 1 K steps
  auto prologue = [&](int u) {
    int tm, tn, z, kb, ke;
    pipe_tile(u, tiles_m, tiles_n, tm, tn, z);
    k_range(z, kb, ke);
    la.setup(A, p.lda, tm * BM, p.M, p.K, tid);
    lb.setup(B, p.ldb, tn * BN, p.N, p.K, tid);
    const int nk = (ke - kb + BK - 1) / BK;
    static_for<S - 1>([&](auto I_) {
      constexpr int I = decltype(I_)::value;
      if (I < nk) {
        la.load(stage(I_), kb + I * BK, ke);
        lb.load(stage_b(I_), kb + I * BK, ke);
      }
    });
    if constexpr (PRE) {
#pragma unroll
      for (int i = 0; i < PRE_I; ++i) load_pre(tm, tn, i);
    }
  };

  constexpr int NST = EARLY ? TM * NQ * (EPI == EPI_GELU ? 2 : 1) : 0;
  // the residual / GELU-input loads a unit's prologue issues after its first
  // K steps' loads: the first step need not wait for them
  constexpr int NPRE = PRE ? PRE_I * NQ : 0;
  static_assert(NST + NPRE + (S - 2) * NLD < 64, "vmcnt range");
  // GELU' epilogue of 128-row tiles in wave rows of 64: the column sums of
  // the outputs (GemmOp::colsum), per lane over its rows of the unit
  constexpr bool CSUM = EPI == EPI_DGELU && PRE && H && BM == 128 && WGM == 2;
  float csum[CSUM ? 8 : 1];
#pragma unroll
  for (int e = 0; e < (CSUM ? 8 : 1); ++e) csum[e] = 0.f;
  f32x16_t acc[TM][TN];
  int round = 0;
  // Unit order. Round-major (pipe_unit): all XCDs work on one window of
  // units at a time, each on new panels every round. XCD-major, for the
  // 128 x 128 GELU epilogue when an XCD's share of the A panels stays in its
  // L2 (at most 2 MB): XCD x owns m-tiles [x tmx, (x + 1) tmx) for the whole
  // launch, keeps their A panels resident and walks the n-tiles from an offset
  // of its own (x n-tiles / 8), so the XCDs do not fetch the same B panel at
  // the same time. Measured on the MLP-in forward at 8192 x 3072 x 768: 59.2
  // -> 55.6 us; on the GELU' input gradient of the same shape and on the
  // 32768-row workload's GEMMs (A shares of 4 MB) no gain, so they keep the
  // round-major order, nor on the 4096 x 1024 x 256 one (K = 256: 2 us
  // slower). Either order covers every tile exactly once.
  const bool xm = EPI == EPI_GELU && BM == 128 && BN == 128 && (tiles_m & 7) == 0 &&
                  units == tiles_m * tiles_n && (nb & 7) == 0 && p.K >= 512 &&
                  (long)(tiles_m >> 3) * BM * p.K * 2 <= (2L << 20);
  auto next_unit = [&](int rd) -> int {
    if (!xm) return pipe_unit(rd, blockIdx.x, nb);
    const int x = blockIdx.x & 7, local = blockIdx.x >> 3, per_xcd = nb >> 3, tmx = tiles_m >> 3;
    const int j = rd * per_xcd + local;
    if (j >= tmx * tiles_n) return units;
    const int tm_ = x * tmx + j % tmx;
    const int tn_ = (j / tmx + x * ((tiles_n + 7) >> 3)) % tiles_n;
    // the unit number pipe_tile maps to (tm_, tn_) (whole groups of 8 m-tiles)
    return (tm_ >> 3) * 8 * tiles_n + tn_ * 8 + (tm_ & 7);
  };
  int u = next_unit(0);
  if (u < units) prologue(u);
  for (; u < units; u = next_unit(++round)) {
    int tm, tn, z, kb, ke;
    pipe_tile(u, tiles_m, tiles_n, tm, tn, z);
    k_range(z, kb, ke);
    const int nk = (ke - kb + BK - 1) / BK;
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int j = 0; j < TN; ++j)
#pragma unroll
        for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;

    for (int it0 = 0; it0 < nk; it0 += S) {
      static_for<S>([&](auto I_) {
        constexpr int I = decltype(I_)::value;
        const int it = it0 + I;
        if (it < nk) {
          // own loads of step it complete (later steps may still be landing),
          // then every wavefront's: the stage is readable, and the stage read
          // at step it - 1 is free
          if (I == 0 && it0 == 0 && EARLY && round > 0) {
            if (it + S - 2 < nk) wait_vmcnt<(S - 2) * NLD + NPRE + NST>();
            else wait_vmcnt<NPRE + NST>();
          } else if (I == 0 && it0 == 0) {
            if (it + S - 2 < nk) wait_vmcnt<(S - 2) * NLD + NPRE>();
            else wait_vmcnt<NPRE>();
          } else if (it + S - 2 < nk) wait_vmcnt<(S - 2) * NLD>();
          else wait_vmcnt<0>();
          lds_barrier();
          const bf16* sa = stage(I_);
          const bf16* sb = stage_b(I_);
          bf16x8_t af[2][TM], bfr[2][TN];
#pragma unroll
          for (int i = 0; i < TM; ++i) af[0][i] = LA::frag(sa, wm * WTM + i * 32, 0, lane);
#pragma unroll
          for (int j = 0; j < TN; ++j) bfr[0][j] = LB::frag(sb, wn * WTN + j * 32, 0, lane);
#pragma unroll
          for (int ks = 0; ks < KS; ++ks) {
            const int f = ks & 1;
            if (ks < 2) {
              // the loads of step it + S - 1 (A during k-step 0, B during
              // k-step 1), spread between the MFMAs; issued even past the
              // last step, where every lane's offset is out of range (zeros
              // into a stage nobody reads), so no branch splits the schedule
              constexpr int NX = (I + S - 1) % S;
              bf16* sx = stage(std::integral_constant<int, NX>{});
              bf16* sxb = stage_b(std::integral_constant<int, NX>{});
              const int kn = it + S - 1 < nk ? kb + (it + S - 1) * BK : ke;
              if (ks == 0) la.load(sx, kn, ke);
              else lb.load(sxb, kn, ke);
            }
            if (ks + 1 < KS) {
#pragma unroll
              for (int i = 0; i < TM; ++i) af[f ^ 1][i] = LA::frag(sa, wm * WTM + i * 32, ks + 1, lane);
#pragma unroll
              for (int j = 0; j < TN; ++j) bfr[f ^ 1][j] = LB::frag(sb, wn * WTN + j * 32, ks + 1, lane);
            }
#pragma unroll
            for (int i = 0; i < TM; ++i)
#pragma unroll
              for (int j = 0; j < TN; ++j)
                acc[i][j] = mfma32<E>(bfr[f][j], af[f][i], acc[i][j]);
            // after each MFMA: one LDS read of the next k-step, one direct
            // load and its address arithmetic
#pragma unroll
            for (int q = 0; q < TM * TN; ++q) {
              __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
              __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
              __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
              __builtin_amdgcn_sched_group_barrier(0x002, 6, 0);
              __builtin_amdgcn_sched_group_barrier(0x004, 2, 0);
            }
            __builtin_amdgcn_sched_barrier(0);
          }
        }
      });
    }
    // Outputs through LDS. Every wavefront is done reading the stages; each
    // owns a 32 x 64 fp32 region of the stage-1 arrays. Pass i writes
    // accumulator rows i*32 .. +31 (element e of tile (i, j): row lane % 32,
    // column j*32 + (e/4)*8 + (lane/32)*4 + e%4), 16-byte chunk c of row r at
    // c ^ (r % 16), reads them back with consecutive lanes on consecutive
    // columns of a row and stores them, so each store instruction writes
    // whole row segments (4 rows x 256 B of fp32, or 8 rows x 128 B of 16-bit
    // values) instead of 16 bytes in each of 32 rows. The last K steps issue
    // loads past the end of K (zeros into a stage nobody reads, possibly
    // stage 1): every wavefront waits for its own before the barrier, so no
    // direct load is still writing the regions. The next unit's first loads
    // (into stage 0) never overlap the region accesses: the compiler's wait
    // counting would hold those until the loads land. Where they follow the
    // stores, the next unit's first wait also waits for those stores (the
    // counter retires in issue order); for 16-bit plain and GELU outputs
    // (EARLY) every pass is read back into registers first, then the loads
    // are issued, then the stores, which the first wait leaves in flight.
    wait_vmcnt<0>();
    lds_barrier();
    static_assert(WTN == 64, "epilogue regions hold 64 columns");
    constexpr int NW = WGM * WGN, REG = 32 * WTN;
    static_assert((NW / 2) * REG * 4 <= LA::ELEMS * 2 && (NW / 2) * REG * 4 <= LB::ELEMS * 2,
                  "epilogue regions fit in stage 1");
    const int un = next_unit(round + 1);
    const long col0 = (long)tn * BN + wn * WTN;
    __amdgpu_buffer_rsrc_t rc, rx;
    // EARLY: the bias of the lane's 8 columns (the same in every pass),
    // loaded once before anything else is in flight (a load per store would
    // wait for the stores before it, the counter retiring in issue order) and
    // added as the outputs of every pass are read back from the regions
    // (plain stores keep them packed, the GELU epilogue in fp32), all before
    // the next unit's loads start. (The other paths load it per chunk: held
    // in registers it measured slower on the wide bias-free GEMMs.)
    constexpr bool EG = EARLY && EPI == EPI_GELU, ES = EARLY && EPI == EPI_STORE;
    float bv[EARLY ? 8 : 1];
    f32x4_t outs[EG ? TM : 1][EG ? 2 * NQ : 1];
    w4_t outp[ES ? TM : 1][ES ? NQ : 1];
    if constexpr (EARLY) {
      const long cl = col0 + (lane % LPR) * CW;
#pragma unroll
      for (int e = 0; e < 8; ++e) bv[e] = 0.f;
      if (p.bias && cl < p.N) ld8_f32(p.bias + cl, bv);
    }
    if constexpr (PRE) {
#pragma unroll
      for (int i = PRE_I; i < TM; ++i) load_pre(tm, tn, i);
    }
    if constexpr (EARLY) {
      // resources from the tile's origin to the last output element
      const long r0 = (long)tm * BM, c0 = (long)tn * BN;
      const long nc = r0 < p.M_out ? ((p.M_out - 1 - r0) * p.ldc + p.N - c0) * 2 : 0;
      rc = __builtin_amdgcn_make_buffer_rsrc(reinterpret_cast<E*>(p.C) + r0 * p.ldc + c0, (short)0,
                                             (int)min(nc, (long)0x7fffffff), 0x00020000);
      if constexpr (EPI == EPI_GELU) {
        const long na = r0 < p.M_out ? ((p.M_out - 1 - r0) * p.ld_aux + p.N - c0) * 2 : 0;
        rx = __builtin_amdgcn_make_buffer_rsrc(reinterpret_cast<E*>(p.aux) + r0 * p.ld_aux + c0, (short)0,
                                               (int)min(na, (long)0x7fffffff), 0x00020000);
      }
    }
    // (the two halves of the wavefronts take the two arrays in separate code
    // paths, so each access has one known LDS object)
    auto epilogue_via = [&](float* __restrict__ reg) {
#pragma unroll
      for (int i = 0; i < TM; ++i) {
        const int rw = lane & 31;
#pragma unroll
        for (int j = 0; j < TN; ++j)
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            const int c = j * 8 + g * 2 + (lane >> 5);
            *reinterpret_cast<f32x4_t*>(reg + rw * 64 + ((c ^ (rw & 15)) << 2)) =
                f32x4_t{acc[i][j][4 * g], acc[i][j][4 * g + 1], acc[i][j][4 * g + 2], acc[i][j][4 * g + 3]};
          }
        f32x4_t out[H ? 2 * NQ : NQ];
#pragma unroll
        for (int q = 0; q < NQ; ++q) {
          const int r = q * RPQ + lane / LPR, c = (lane % LPR) * (CW / 4);
          out[H ? 2 * q : q] = *reinterpret_cast<const f32x4_t*>(reg + r * 64 + ((c ^ (r & 15)) << 2));
          if constexpr (H)
            out[2 * q + 1] = *reinterpret_cast<const f32x4_t*>(reg + r * 64 + (((c + 1) ^ (r & 15)) << 2));
        }
        const long row0 = (long)tm * BM + wm * WTM + i * 32;
#pragma unroll
        for (int q = 0; q < NQ; ++q) {
          const long row = row0 + q * RPQ + lane / LPR, col = col0 + (lane % LPR) * CW;
          if constexpr (EG) {
            outs[i][2 * q] = out[2 * q] + f32x4_t{bv[0], bv[1], bv[2], bv[3]};
            outs[i][2 * q + 1] = out[2 * q + 1] + f32x4_t{bv[4], bv[5], bv[6], bv[7]};
            continue;
          } else if constexpr (ES) {
            const f32x4_t lo = out[2 * q], hi = out[2 * q + 1];
            outp[i][q] = w4_t{H16<E>::pack(lo[0] + bv[0], lo[1] + bv[1]), H16<E>::pack(lo[2] + bv[2], lo[3] + bv[3]),
                              H16<E>::pack(hi[0] + bv[4], hi[1] + bv[5]), H16<E>::pack(hi[2] + bv[6], hi[3] + bv[7])};
            continue;
          }
          if (row >= p.M_out || col >= p.N) continue;
          if constexpr (PRE && EPI == EPI_DGELU) {
            const f32x4_t lo = out[2 * q], hi = out[2 * q + 1];
            const uint4 u = pre[i][q];
            float v[8] = {lo[0] * H16<E>::lo(u.x), lo[1] * H16<E>::hi(u.x),
                          lo[2] * H16<E>::lo(u.y), lo[3] * H16<E>::hi(u.y),
                          hi[0] * H16<E>::lo(u.z), hi[1] * H16<E>::hi(u.z),
                          hi[2] * H16<E>::lo(u.w), hi[3] * H16<E>::hi(u.w)};
            st8_h<E>(reinterpret_cast<E*>(p.C) + row * p.ldc + col, v);
            if constexpr (CSUM) {
#pragma unroll
              for (int e = 0; e < 8; ++e) csum[e] += v[e];
            }
          } else if constexpr (PRE && EPI == EPI_RESID) {
            f32x4_t v = out[q];
            if (p.bias) v += *reinterpret_cast<const f32x4_t*>(p.bias + col);
            v += __builtin_bit_cast(f32x4_t, pre[i][q]);
            *reinterpret_cast<f32x4_t*>(reinterpret_cast<float*>(p.C) + row * p.ldc + col) = v;
          } else if constexpr (H) {
            const f32x4_t lo = out[2 * q], hi = out[2 * q + 1];
            float v[8] = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
            epilogue8<EPI, TC, E>(p, row, col, v, z);
          } else {
            epilogue4<EPI, TC, E>(p, row, col, out[q], z);
          }
        }
      }
    };
    constexpr std::integral_constant<int, 1> I1{};
    if (wave < NW / 2) epilogue_via(reinterpret_cast<float*>(stage(I1)) + wave * REG);
    else epilogue_via(reinterpret_cast<float*>(stage_b(I1)) + (wave - NW / 2) * REG);
    if constexpr (CSUM) {
      // lanes l, l + LPR, ... hold the same 8 columns: a fixed xor tree over
      // them, then the wave row's 64-row sums of its 64 columns
#pragma unroll
      for (int o = LPR; o < 64; o <<= 1)
#pragma unroll
        for (int e = 0; e < 8; ++e) csum[e] += __shfl_xor(csum[e], o, 64);
      if (p.colsum && lane < LPR) {
        const long col = col0 + lane * CW;
        if (col < p.N) {
          float* d = p.colsum + ((long)tm * WGM + wm) * p.N + col;
          *reinterpret_cast<f32x4_t*>(d) = f32x4_t{csum[0], csum[1], csum[2], csum[3]};
          *reinterpret_cast<f32x4_t*>(d + 4) = f32x4_t{csum[4], csum[5], csum[6], csum[7]};
        }
      }
#pragma unroll
      for (int e = 0; e < 8; ++e) csum[e] = 0.f;
    }
    if constexpr (!EARLY) {
      if (un < units) prologue(un);
    } else {
      // (the bias loads are done by now; an explicit wait tells the compiler
      // so, else the register uses it moves past the next loads wait for them)
      wait_vmcnt<0>();
      if (un < units) prologue(un);
      const int rows = (int)min((long)BM, p.M_out - (long)tm * BM), cols = (int)min((long)BN, p.N - (long)tn * BN);
      const int ldc = (int)p.ldc, ldx = (int)p.ld_aux;
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int q = 0; q < NQ; ++q) {
          const int lr = wm * WTM + i * 32 + q * RPQ + lane / LPR, lc = wn * WTN + (lane % LPR) * CW;
          const bool ok = lr < rows && lc < cols;
          const unsigned oc = ok ? (unsigned)((lr * ldc + lc) * 2) : kOutOfRange;
          if constexpr (ES) {
            __builtin_amdgcn_raw_buffer_store_b128(outp[i][q], rc, (int)oc, 0, 0);
          } else {
            const f32x4_t lo = outs[i][2 * q], hi = outs[i][2 * q + 1];
            const float u[8] = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
            float g[8], d[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) gelu_and_grad(u[e], g[e], d[e]);
            bst8_h<E>(rc, oc, d);
            bst8_h<E>(rx, ok ? (unsigned)((lr * ldx + lc) * 2) : kOutOfRange, g);
          }
        }
    }
  }
  // no direct load may still be writing LDS when the workgroup ends
  wait_vmcnt<0>();
}

// --------------------------------------------- persistent K-split GEMM
// One block of eight wavefronts per CU on a 128 x (64 TN) tile. The
// wavefronts form two groups of four, each group a 2 x 2 grid of 64 x 32 TN
// wave tiles over the whole block tile; every K step of 64 is split between
// the groups (group g takes k-slices 2g and 2g + 1), so each SIMD runs one
// wavefront of each group: while one waits on the step's barrier or its
// fragment reads, the other issues matrix instructions. A second wavefront
// per SIMD would otherwise need a tile twice as large, and the tile count of
// the 768-wide outputs at 8192 rows (exactly one 128 x 192 tile per CU; 3 and
// 4 per CU for the 2304- and 3072-wide ones) would no longer fill the chip.
// Operands arrive by direct-to-LDS loads in three stages (two K steps ahead),
// one LDS array per stage and operand as in the persistent kernel above.
// At the end of a tile the groups add their partial sums through LDS: group g
// keeps its wave tile's rows 32 g .. 32 g + 31 and receives the other group's
// partial sums of them (a + b, the same in either order: the result does not
// depend on which group arrives first), then stores those 32 rows straight
// from registers; the residual or GELU'(u) of those rows is loaded ahead,
// with the tile's first K steps.
//
// GROUP: the units of several GEMMs of the same layout and epilogue in one
// launch (table tab, units numbered GEMM after GEMM), each unit one whole
// tile over all of K; the arguments of a unit's GEMM are read from the table.
template <int TN, int S, bool AK, bool BKC, int EPI, typename TC, typename E, bool GROUP = false>
__global__ void __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2, 2)))
    gemm16_ksplit_kernel(GemmArgs p_in, int units, int tiles_m, int tiles_n,
                         const GemmGroupEntry* __restrict__ tab) {
  constexpr int BM = 128, TM = 2, WTM = 64, WTN = 32 * TN, BN = 2 * WTN, BK = 64, NT = 512;
  static_assert(S == 3 || S == 4, "three or four stages");
  using LA = PTile<BM, AK, NT, BK>;
  using LB = PTile<BN, BKC, NT, BK>;
  constexpr int NLD = LA::NI + LB::NI;  // load instructions per wavefront per K step
  constexpr bool H = sizeof(TC) == 2;
  // epilogue operands, 4 columns of a row per chunk, TN * 4 chunks per lane:
  // the 16-bit GELU'(u) (8 bytes a chunk) is loaded with the tile's first
  // K steps; the fp32 residual (16 bytes a chunk: 48 more registers through
  // the K loop would spill) right after the K loop, its latency partly
  // hidden by the exchange of the partial sums
  constexpr bool PRE = EPI == EPI_DGELU;
  constexpr bool POST = EPI == EPI_RESID;
  constexpr int NPRE = PRE ? TN * 4 : 0;
  static_assert(NPRE + NLD < 64, "vmcnt range");
  // exchange regions: 32 x WTN fp32 per wavefront, in the stage arrays (two
  // per B stage array; with three stages the last two in A stages 0 and 1),
  // and the tile's bias in A stage S - 1 (S = 4) or 2
  constexpr int REG = 32 * WTN;  // floats
  static_assert(2 * REG * 4 <= LB::ELEMS * 2 && REG * 4 <= LA::ELEMS * 2, "exchange regions fit");

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int grp = wave >> 2, wm = (wave >> 1) & 1, wn = wave & 1;
  GemmArgs p = p_in;
  const int nb = gridDim.x;
  // the tile (tm, tn) and K slice z of unit u; with GROUP also its GEMM's
  // arguments into p (units are visited in increasing order, so the table
  // index only moves forward)
  int gi = 0;
  auto locate = [&](int u, int& tm, int& tn, int& z) {
    if constexpr (GROUP) {
      while (u >= tab[gi + 1].first_unit) ++gi;
      p = tab[gi].a;
      pipe_tile(u - tab[gi].first_unit, tab[gi].tiles_m, tab[gi].tiles_n, tm, tn, z);
    } else {
      pipe_tile(u, tiles_m, tiles_n, tm, tn, z);
    }
  };
  auto sa = [](auto I_) -> bf16* { return lds_stage<2 * decltype(I_)::value, LA::ELEMS>(); };
  auto sb = [](auto I_) -> bf16* { return lds_stage<2 * decltype(I_)::value + 1, LB::ELEMS>(); };
  // region r of the exchange as an fp32 pointer into one known LDS array
  // (waves 0..5: the B stage arrays, two per array; 6, 7: A stages 0, 1)
  auto with_region = [&](int r, auto&& f) {
    constexpr std::integral_constant<int, 0> I0{};
    constexpr std::integral_constant<int, 1> I1{};
    constexpr std::integral_constant<int, 2> I2{};
    constexpr std::integral_constant<int, S == 4 ? 3 : 0> I3{};
    switch (r) {
      case 0: f(reinterpret_cast<float*>(sb(I0))); break;
      case 1: f(reinterpret_cast<float*>(sb(I0)) + REG); break;
      case 2: f(reinterpret_cast<float*>(sb(I1))); break;
      case 3: f(reinterpret_cast<float*>(sb(I1)) + REG); break;
      case 4: f(reinterpret_cast<float*>(sb(I2))); break;
      case 5: f(reinterpret_cast<float*>(sb(I2)) + REG); break;
      case 6:
        if constexpr (S == 4) f(reinterpret_cast<float*>(sb(I3)));
        else f(reinterpret_cast<float*>(sa(I0)));
        break;
      default:
        if constexpr (S == 4) f(reinterpret_cast<float*>(sb(I3)) + REG);
        else f(reinterpret_cast<float*>(sa(I1)));
        break;
    }
  };
  // the tile's bias in a stage array no exchange region uses
  auto bias_lds = [&]() -> float* {
    return reinterpret_cast<float*>(sa(std::integral_constant<int, S == 4 ? S - 1 : 2>{}));
  };

  LA la;
  LB lb;
  // lane's output chunk (j, c4): row lane % 32 of the group's 32 rows,
  // columns j * 32 + c4 * 8 + (lane / 32) * 4 .. + 3 of the wave tile
  const int lrow = wm * WTM + grp * 32 + (lane & 31);
  auto lcol = [&](int j, int c4) { return wn * WTN + j * 32 + c4 * 8 + (lane >> 5) * 4; };
  typedef unsigned int w2_t __attribute__((ext_vector_type(2)));
  typedef std::conditional_t<EPI == EPI_DGELU, w2_t, uint4> pre_t;
  pre_t pre[PRE || POST ? TN * 4 : 1];
  // the tile's bias: loaded by wavefront 0 with the tile's first loads, kept
  // in LDS for the epilogue
  constexpr bool BIAS = EPI == EPI_STORE || EPI == EPI_RESID || EPI == EPI_GELU;
  static_assert(BN * 4 <= LA::ELEMS * 2, "the bias fits in an A stage");
  f32x4_t bias_r = f32x4_t{0.f, 0.f, 0.f, 0.f};
  auto load_pre = [&](int tm, int tn) {
    constexpr int ES = EPI == EPI_DGELU ? 2 : 4;
    const long r0 = (long)tm * BM, c0 = (long)tn * BN;
    const long ld = EPI == EPI_DGELU ? p.ld_aux : p.ldr;
    const char* base = EPI == EPI_DGELU ? reinterpret_cast<const char*>(p.aux) : reinterpret_cast<const char*>(p.R);
    const long n = r0 < p.M_out ? ((p.M_out - 1 - r0) * ld + p.N - c0) * ES : 0;
    const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(base + (r0 * ld + c0) * ES), (short)0, (int)min(n, (long)0x7fffffff), 0x00020000);
    const int ldi = (int)ld, rows = (int)min((long)BM, p.M_out - r0), cols = (int)min((long)BN, p.N - c0);
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int c4 = 0; c4 < 4; ++c4) {
        const int lc = lcol(j, c4);
        const int off = lrow < rows && lc < cols ? (lrow * ldi + lc) * ES : (int)kOutOfRange;
        if constexpr (ES == 4) {
          const w4_t w = __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0);
          pre[j * 4 + c4] = make_uint4(w[0], w[1], w[2], w[3]);
        } else {
          pre[j * 4 + c4] = __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, 0);
        }
      }
  };
  auto prologue = [&](int tm, int tn, int z) {
    const bf16* A = reinterpret_cast<const bf16*>(p.A);
    const bf16* B = reinterpret_cast<const bf16*>(p.B);
    const int kb = z * p.k_split, ke = min(p.K, kb + p.k_split);
    if constexpr (BIAS) {
      // the tile's bias, by wavefront 0 ahead of the stage loads (the first
      // K step waits for it with them); zero where absent, so the epilogue
      // adds it unconditionally. (A load inside the K loop would make the
      // compiler wait for every outstanding load before the register's
      // later uses.)
      if (wave == 0 && lane < BN / 4) {
        const long col = (long)tn * BN + lane * 4;
        bias_r = p.bias && col < p.N ? *reinterpret_cast<const f32x4_t*>(p.bias + col)
                                     : f32x4_t{0.f, 0.f, 0.f, 0.f};
      }
    }
    la.setup(A, p.lda, tm * BM, p.M, p.K, tid);
    lb.setup(B, p.ldb, tn * BN, p.N, p.K, tid);
    // the first S - 1 K steps, issued even past the end of K (zeros into a
    // stage nobody reads), so every wavefront has the same loads in flight
    static_for<S - 1>([&](auto I_) {
      constexpr int I = decltype(I_)::value;
      const int k0 = kb + I * BK < ke ? kb + I * BK : ke;
      la.load(sa(I_), k0, ke);
      lb.load(sb(I_), k0, ke);
    });
    if constexpr (PRE) load_pre(tm, tn);
  };

  f32x16_t acc[TM][TN];
  int round = 0;
  int u = pipe_unit(0, blockIdx.x, nb);
  for (; u < units; u = pipe_unit(++round, blockIdx.x, nb)) {
    int tm, tn, z;
    locate(u, tm, tn, z);
    const int kb = z * p.k_split, ke = min(p.K, kb + p.k_split);
    const int nk = (ke - kb + BK - 1) / BK;
    prologue(tm, tn, z);
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int j = 0; j < TN; ++j)
#pragma unroll
        for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;

    // One K step at stage I (it = the step's index).
    auto kstep = [&](auto I_, int it) {
      constexpr int I = decltype(I_)::value;
      // this wavefront's loads of step it have landed (the S - 2 later
      // steps' may still be landing; the epilogue operands, issued after
      // the first S - 1 steps, before step 2), then every wavefront's:
      // stage I is readable, and the stage read at step it - 1 is free
      if (it < 2) wait_vmcnt<(S - 2) * NLD + NPRE>();
      else wait_vmcnt<(S - 2) * NLD>();
      lds_barrier();
      const bf16* a_s = sa(I_);
      const bf16* b_s = sb(I_);
      bf16x8_t af[2][TM], bfr[2][TN];
#pragma unroll
      for (int i = 0; i < TM; ++i) af[0][i] = LA::frag(a_s, wm * WTM + i * 32, 2 * grp, lane);
#pragma unroll
      for (int j = 0; j < TN; ++j) bfr[0][j] = LB::frag(b_s, wn * WTN + j * 32, 2 * grp, lane);
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
        // the loads of step it + S - 1 into the stage read at step it - 1
        // (A during the first k-slice, B during the second)
        constexpr int NX = (I + S - 1) % S;
        const int kn = it + S - 1 < nk ? kb + (it + S - 1) * BK : ke;
        if (kk == 0) la.load(sa(std::integral_constant<int, NX>{}), kn, ke);
        else lb.load(sb(std::integral_constant<int, NX>{}), kn, ke);
        if (kk == 0) {
#pragma unroll
          for (int i = 0; i < TM; ++i) af[1][i] = LA::frag(a_s, wm * WTM + i * 32, 2 * grp + 1, lane);
#pragma unroll
          for (int j = 0; j < TN; ++j) bfr[1][j] = LB::frag(b_s, wn * WTN + j * 32, 2 * grp + 1, lane);
        }
#pragma unroll
        for (int i = 0; i < TM; ++i)
#pragma unroll
          for (int j = 0; j < TN; ++j) acc[i][j] = mfma32<E>(bfr[kk][j], af[kk][i], acc[i][j]);
#pragma unroll
        for (int q = 0; q < TM * TN; ++q) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
          __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
          __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
          __builtin_amdgcn_sched_group_barrier(0x002, 4, 0);
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    };
    // Whole groups of S steps in the loop and the remaining steps after it:
    // with a conditional step inside the loop, the wait-count analysis would
    // see a path on which the stage about to be read was loaded last, and wait
    // for every outstanding load before its reads.
    int it0 = 0;
    for (; it0 + S <= nk; it0 += S) static_for<S>([&](auto I_) { kstep(I_, it0 + decltype(I_)::value); });
    static_for<S - 1>([&](auto I_) {
      if (it0 + decltype(I_)::value < nk) kstep(I_, it0 + decltype(I_)::value);
    });
    // no direct load is still writing a stage and every wavefront is done
    // reading them: the stages become the exchange regions; the tile's bias
    // (loaded by wavefront 0 with the tile's first loads) goes to LDS, so
    // that the epilogue's bias reads do not wait for its stores
    wait_vmcnt<0>();
    lds_barrier();
    if constexpr (BIAS) {
      if (wave == 0 && lane < BN / 4) *reinterpret_cast<f32x4_t*>(bias_lds() + lane * 4) = bias_r;
    }
    if constexpr (POST) load_pre(tm, tn);
    const long r0 = (long)tm * BM, c0 = (long)tn * BN;
    const int rows = (int)min((long)BM, p.M_out - r0), cols = (int)min((long)BN, p.N - c0);
    const int ldc = (int)p.ldc, ldx = (int)p.ld_aux;
    // stores through resources from the tile's origin (an offset past the
    // range is dropped)
    auto rsrc_of = [&](void* base, long ld, int es) {
      const long n = r0 < p.M_out ? ((p.M_out - 1 - r0) * ld + p.N - c0) * es : 0;
      return __builtin_amdgcn_make_buffer_rsrc(reinterpret_cast<char*>(base) + (r0 * ld + c0) * es, (short)0,
                                               (int)min(n, (long)0x7fffffff), 0x00020000);
    };
    void* cbase = EPI == EPI_PARTIAL ? static_cast<void*>(reinterpret_cast<float*>(p.C) + (long)z * p.split_stride)
                                     : p.C;
    const __amdgpu_buffer_rsrc_t rc = rsrc_of(cbase, p.ldc, H ? 2 : 4);
    const __amdgpu_buffer_rsrc_t rx = EPI == EPI_GELU ? rsrc_of(p.aux, p.ld_aux, 2) : rc;
    typedef unsigned int w2_t __attribute__((ext_vector_type(2)));
    // the epilogue of chunk q (j = q / 4, c4 = q % 4) with its summed value v
    auto store = [&](int q, f32x4_t v) {
      const int lc = lcol(q >> 2, q & 3);
      const bool ok = lrow < rows && lc < cols;
      if constexpr (BIAS) v += *reinterpret_cast<const f32x4_t*>(bias_lds() + lc);
      if constexpr (EPI == EPI_RESID) v += __builtin_bit_cast(f32x4_t, pre[q]);
      if constexpr (EPI == EPI_DGELU) {
        const w2_t uu = pre[q];
        v[0] *= H16<E>::lo(uu[0]);
        v[1] *= H16<E>::hi(uu[0]);
        v[2] *= H16<E>::lo(uu[1]);
        v[3] *= H16<E>::hi(uu[1]);
      }
      if constexpr (H) {
        f32x4_t g;
        if constexpr (EPI == EPI_GELU) {
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            float ge, de;
            gelu_and_grad(v[e], ge, de);
            g[e] = ge;
            v[e] = de;
          }
        }
        const w2_t w = w2_t{H16<E>::pack(v[0], v[1]), H16<E>::pack(v[2], v[3])};
        __builtin_amdgcn_raw_buffer_store_b64(w, rc, ok ? (lrow * ldc + lc) * 2 : (int)kOutOfRange, 0, 0);
        if constexpr (EPI == EPI_GELU) {
          const w2_t gw = w2_t{H16<E>::pack(g[0], g[1]), H16<E>::pack(g[2], g[3])};
          __builtin_amdgcn_raw_buffer_store_b64(gw, rx, ok ? (lrow * ldx + lc) * 2 : (int)kOutOfRange, 0, 0);
        }
      } else {
        __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(w4_t, v), rc,
                                               ok ? (lrow * ldc + lc) * 4 : (int)kOutOfRange, 0, 0);
      }
    };
    // (the group is uniform over a wavefront: one code path per group keeps
    // the accumulator indices compile-time constants; both paths meet the
    // same two barriers)
    auto exchange = [&](auto G_) {
      constexpr int G = decltype(G_)::value;
      with_region(wave, [&](float* __restrict__ reg) {
#pragma unroll
        for (int j = 0; j < TN; ++j)
#pragma unroll
          for (int c4 = 0; c4 < 4; ++c4) {
            const f32x16_t& a = acc[G ^ 1][j];
            *reinterpret_cast<f32x4_t*>(reg + ((j * 4 + c4) * 64 + lane) * 4) =
                f32x4_t{a[4 * c4], a[4 * c4 + 1], a[4 * c4 + 2], a[4 * c4 + 3]};
          }
      });
      lds_barrier();
      with_region(wave ^ 4, [&](const float* __restrict__ reg) {
#pragma unroll
        for (int j = 0; j < TN; ++j)
#pragma unroll
          for (int c4 = 0; c4 < 4; ++c4) {
            const f32x16_t& a = acc[G][j];
            store(j * 4 + c4, f32x4_t{a[4 * c4], a[4 * c4 + 1], a[4 * c4 + 2], a[4 * c4 + 3]} +
                                  *reinterpret_cast<const f32x4_t*>(reg + ((j * 4 + c4) * 64 + lane) * 4));
          }
      });
      // the regions and the bias are read: the next tile's loads may
      // overwrite the stages
      lds_barrier();
    };
    if (grp == 0) exchange(std::integral_constant<int, 0>{});
    else exchange(std::integral_constant<int, 1>{});
  }
  // no direct load may still be writing LDS when the workgroup ends
  wait_vmcnt<0>();
}

// ------------------------------------------------------------- dispatch
static GemmArgs make_args(const GemmOp& op) {
  GemmArgs a;
  a.A = op.A; a.lda = op.lda; a.B = op.B; a.ldb = op.ldb; a.C = op.C; a.ldc = op.ldc;
  a.bias = op.bias; a.R = op.R; a.ldr = op.ldr; a.aux = op.aux; a.ld_aux = op.ld_aux;
  a.M = op.M; a.N = op.N; a.K = op.K; a.k_split = op.K; a.split_stride = 0;
  a.M_out = op.M_out > 0 && op.M_out < op.M ? op.M_out : op.M;
  a.colsum = op.colsum;
  return a;
}

// Bytes an operand spans from its first element: rows of ld elements,
// the last one `width` long (K-contiguous: M or N rows of K; otherwise K
// rows of M or N).
static long span_bytes(long rows, long ld, long width, long elem) {
  return rows <= 0 ? 0 : ((rows - 1) * ld + width) * elem;
}

static bool check_16(const GemmOp& op) {
  if (op.lda % 8 || op.ldb % 8) return false;
  // the operand loaders address each operand through a buffer resource with
  // a 32-bit range and 32-bit per-lane byte offsets
  const long a_span = op.a_kc ? span_bytes(op.M, op.lda, op.K, 2) : span_bytes(op.K, op.lda, op.M, 2);
  const long b_span = op.b_kc ? span_bytes(op.N, op.ldb, op.K, 2) : span_bytes(op.K, op.ldb, op.N, 2);
  if (a_span > 0x7fffffffL || b_span > 0x7fffffffL) return false;
  // epilogue operands and outputs are addressed by 32-bit byte offsets within
  // a tile of up to 256 rows
  const long ld_max = std::max(op.ldc, std::max(op.R ? op.ldr : 0L, op.aux ? op.ld_aux : 0L));
  if (256L * ld_max * 4 >= (1L << 31)) return false;
  // 8-column epilogue chunks: N and every leading dimension of the outputs
  if (op.N % 8 || op.ldc % 8 || (op.R && op.ldr % 8) || (op.aux && op.ld_aux % 8)) return false;
  if ((op.a_kc || op.b_kc) && op.K % 8) return false;
  if (!op.a_kc && op.M % 8) return false;
  if (!op.b_kc && op.N % 8) return false;
  return true;
}

// Tile configurations: 1 = gemm16_kernel 128 x 128 (4 wavefronts of 64 x 64,
// two blocks per CU, register-staged loads); 11 = gemm16_pipe_kernel,
// persistent 256 x 256 (8 wavefronts of 128 x 64, two per SIMD, one block per
// CU); 12 = gemm16_pipe_kernel, persistent 128 x 128 (4 wavefronts of 64 x 64,
// two blocks per CU); 14 = the same at 192 x 128 (wavefronts of 96 x 64, two
// blocks per CU in 160 KB of LDS), K-contiguous operands and a plain store.
// 15, 16 = gemm16_ksplit_kernel, persistent 128 x 192 and 128 x 128 (one
// block of eight wavefronts per CU, the K step split between two groups of
// four).
constexpr int kCfgSmall = 1, kCfgPipe = 11, kCfgPipe128 = 12, kCfgPipe192 = 14;
constexpr int kCfgKs192 = 15, kCfgKs128 = 16;

static bool is_ksplit(int cfg) { return cfg == kCfgKs192 || cfg == kCfgKs128; }

static int tiles_of(const GemmOp& op, int cfg) {
  int TMr = 128, TNc = 128;
  if (cfg == kCfgPipe) TMr = TNc = 256;
  else if (cfg == kCfgPipe192) TMr = 192;
  else if (cfg == kCfgKs192) TNc = 192;
  return ((op.M + TMr - 1) / TMr) * ((op.N + TNc - 1) / TNc);
}

// Compute units of the current device (the persistent grid's size).
static int device_cus() {
  static int n[64] = {0};
  int d = 0;
  if (hipGetDevice(&d) != hipSuccess || d < 0 || d >= 64) return 256;
  if (!n[d]) {
    int v = 0;
    n[d] = (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, d) == hipSuccess && v > 0) ? v : 256;
  }
  return n[d];
}

// Configurations a caller may ask for (GemmOp::cfg) for an op: every
// configuration runs every layout and epilogue except the 192 x 128 one,
// which takes K-contiguous operands and a plain 16-bit store only.
static bool cfg_allowed(const GemmOp& op, int cfg) {
  if (cfg == kCfgSmall || cfg == kCfgPipe || cfg == kCfgPipe128 || is_ksplit(cfg)) return true;
  if (cfg == kCfgPipe192) return op.a_kc && op.b_kc && op.epi == EPI_STORE && !op.c_f32;
  return false;
}

// K slices of a K-split op: the most units that still run in one round of
// the persistent grid (one block per CU), with at least 512 K-values per
// slice; the fewest slices among equal fills.
static int ksplit_slices(const GemmOp& op, int cfg) {
  const int cus = device_cus(), tiles = tiles_of(op, cfg);
  int best = 1;
  for (int s = 2; s <= 16 && op.K / s >= 512; ++s)
    if ((long)tiles * s <= cus) best = s;
  return best;
}
static double ksplit_round_fill(const GemmOp& op, int cfg) {
  const int cus = device_cus();
  const long u = (long)tiles_of(op, cfg) * ksplit_slices(op, cfg);
  return (double)u / (double)(((u + cus - 1) / cus) * cus);
}

static int pick_cfg(const GemmOp& op) {
  if (op.cfg > 0) return op.cfg;
  // Measured on the step's shapes: the persistent 256 x 256 kernel wins on
  // the vocabulary projection's forward (very wide N) and weight gradient
  // (very tall M), and on the projections of the 32768-token workload (M =
  // 32768, 512-2048 wide); 128 x 128 at two blocks per CU on most others:
  // the direct-load persistent kernel (6-12% faster), except for the
  // residual epilogue, whose fp32 operand the register-staged kernel loads
  // ahead more fully (the persistent one holds only the first of its two
  // passes through the K loop; 7% slower).
  const int mn_max = op.M > op.N ? op.M : op.N, mn_min = op.M < op.N ? op.M : op.N;
  // Weight gradients of the 768-wide model's blocks (both operands M/N-
  // contiguous, K = the token count, outputs of 768 x 768 to 768 x 3072): the
  // K-split kernel with as many K slices as fill the CUs in one round
  // (gemm16_splits). Measured at 8192 tokens: the MLP weight gradients 50 us
  // (128 x 192 tiles, 2 slices) against 56-58 us for 256 x 256 tiles in 7
  // slices, the QKV one 40 us (128 x 192, 3 slices) against 45 us for 128 x
  // 128 tiles in 4 slices of two blocks per CU, the attention-output one
  // 22 us (128 x 128, 6-7 slices) against 26 us; several rounds of slices
  // measured slower (no overlap of one unit's partial store with the next
  // unit's loads). 128 x 192 tiles where they fill at least 70% of the CUs.
  // (The same at the smaller widths of the other workloads, 128-512: there
  // 128 x 128 tiles, unless the width is a multiple of 192: 2x faster than
  // the split 256 x 256 or 128 x 128 kernels at 128-wide outputs, 5-45% at
  // 512-wide ones.)
  if (!op.a_kc && !op.b_kc && op.K >= 4096 && mn_min >= 128 && mn_max <= 4096 && op.colsum == nullptr)
    return op.N % 192 == 0 && ksplit_round_fill(op, kCfgKs192) >= 0.7 ? kCfgKs192 : kCfgKs128;
  // Outputs 128 or fewer columns wide over many rows (the 128-wide model's
  // projections to d_model): 128 x 128 tiles (a 256-wide tile would be half
  // empty), K-split and in one round of slices when K is long (its
  // vocabulary input and weight gradients: 52 and 50 us against 67 and 70
  // us on 256 x 256 tiles), else two blocks per CU (10 against 22 us on the
  // MLP-out forward).
  if (op.N <= 128 && op.M >= 4096) return op.K >= 4096 ? kCfgKs128 : kCfgPipe128;
  // Outputs whose 128 x 192 tiles fill the CUs in exactly one round (the
  // 768-wide outputs at 8192 rows, including the vocabulary projection's
  // input gradient, whose K of 50304 then needs no split): the K-split
  // kernel, one tile per CU (measured 10-30% faster than the 128 x 128 or
  // split 256 x 256 tiles there; with several tiles per CU it is slower).
  {
    const int cus = device_cus(), t = tiles_of(op, kCfgKs192);
    if (t <= cus && 10 * t >= 9 * cus && op.K >= 512 && op.colsum == nullptr) return kCfgKs192;
  }
  // the GELU' input gradient: the 128 x 128 kernel, whose epilogue also
  // writes the bias gradient's partial column sums (6% faster than 256 x 256
  // at 32768 x 2048 before counting the separate column-sum pass it saves)
  if (op.epi == EPI_DGELU && op.M >= 4096) return kCfgPipe128;
  // (16384 rows alone do not make a 256-row tile pay: at 16384 x 384 and x
  // 512 over K = 128 the 256 x 256 tiles took 12.8 and 19.8 us, the 192 x 128
  // and 128 x 128 ones below 10.3 and 12.1)
  if (op.M >= 32768 || op.N >= 16384 || op.K >= 16384 || (op.M >= 16384 && op.N >= 4096)) return kCfgPipe;
  if (op.K >= 8192 && mn_max >= 3072 && mn_max <= 4096 && mn_min <= 1024) return kCfgPipe;
  if (op.epi == EPI_RESID) return kCfgSmall;
  // the QKV projection (both operands K-contiguous, a plain store): 192 x 128
  // tiles measured 9% faster there (and slower with the GELU or residual
  // epilogues)
  if (op.a_kc && op.b_kc && op.epi == EPI_STORE && op.M >= 4096 && !op.c_f32) return kCfgPipe192;
  return kCfgPipe128;
}

int gemm16_colsum_rows(const GemmOp& op) {
  // the persistent 128 x 128 kernel's GELU' epilogue, in one K slice
  if (op.epi != EPI_DGELU || (op.M_out > 0 && op.M_out < op.M)) return 0;
  if (pick_cfg(op) != kCfgPipe128 || gemm16_splits(op) != 1) return 0;
  return 2 * ((op.M + 127) / 128);
}

int gemm16_splits(const GemmOp& op) {
  if (op.force_split > 0) return op.force_split;
  const int cfg = pick_cfg(op);
  const int tiles = tiles_of(op, cfg);
  if (is_ksplit(cfg)) return ksplit_slices(op, cfg);
  if (cfg == kCfgPipe) {
    // persistent grid of one block per CU: pick the K split whose work units
    // fill the last round best (smallest split within 10% of the best fill),
    // with at least 512 K-values per slice
    const int cus = device_cus();
    auto fill = [&](int s) {
      const long u = (long)tiles * s;
      return (double)u / (double)(((u + cus - 1) / cus) * cus);
    };
    double best = fill(1);
    for (int s = 2; s <= 16 && op.K / s >= 512; ++s) best = fill(s) > best ? fill(s) : best;
    for (int s = 1; s <= 16; ++s)
      if ((s == 1 || op.K / s >= 512) && fill(s) >= 0.9 * best) return s;
    return 1;
  }
  // split K when the tile grid cannot fill the 256 compute units and K is
  // long; for a few rows (one token per sequence when generating) each tile
  // is a short latency-bound pass, so slices go down to 128 K-values
  const int kmin = op.M <= 64 ? 128 : 512;
  int s = 1;
  while (tiles * s < 256 && op.K / (s * 2) >= kmin) s *= 2;
  return s;
}

// OCC: waves per SIMD the kernel is compiled for; blocks per CU = 4 OCC /
// (WGM WGN), and the persistent grid holds that many blocks per CU.
template <int BM, int BN, int WGM, int WGN, int BK, int S, int OCC, bool AK, bool BKC, int EPI, typename TC,
          typename E>
static void launch_pipe(const GemmArgs& a, int splits, hipStream_t s) {
  const int tiles_m = (a.M + BM - 1) / BM, tiles_n = (a.N + BN - 1) / BN;
  const int units = tiles_m * tiles_n * splits;
  constexpr int per_cu = 4 * OCC / (WGM * WGN) > 0 ? 4 * OCC / (WGM * WGN) : 1;
  int nb = device_cus() * per_cu;
  if (units < nb) nb = units;
  nb = (nb + 7) / 8 * 8;  // whole XCD rounds
  hipLaunchKernelGGL((gemm16_pipe_kernel<BM, BN, WGM, WGN, BK, S, OCC, AK, BKC, EPI, TC, E>), dim3(nb),
                     dim3(WGM * WGN * 64), 0, s, a, units, tiles_m, tiles_n);
}

template <int BM, int BN, int WGM, int WGN, bool AK, bool BKC, int EPI, typename TC, typename E>
static void launch_small(const GemmArgs& a, int splits, hipStream_t s) {
  const int units = ((a.M + BM - 1) / BM) * ((a.N + BN - 1) / BN) * splits;
  // Measured on the step's shapes: the GELU epilogue (two outputs, no loaded
  // operand) and the split-K partials gain from a persistent grid (as many
  // blocks as fit on the CUs at once), whose next-unit loads overlap the
  // epilogue; the other epilogues run one block per unit.
  constexpr bool persist = EPI == EPI_GELU || EPI == EPI_PARTIAL;
  constexpr int per_cu = (160 * 1024) / (2 * 2 * 64 * (BM + BN)) > 0 ? (160 * 1024) / (2 * 2 * 64 * (BM + BN)) : 1;
  int nb = persist ? device_cus() * per_cu : units;
  if (units < nb) nb = units;
  nb = (nb + 7) / 8 * 8;  // whole XCD rounds
  hipLaunchKernelGGL((gemm16_kernel<BM, BN, WGM, WGN, AK, BKC, EPI, TC, E>), dim3(nb), dim3(WGM * WGN * 64), 0, s,
                     a, units);
}

template <int TN, int S, bool AK, bool BKC, int EPI, typename TC, typename E>
static void launch_ksplit(const GemmArgs& a, int splits, hipStream_t s) {
  const int tiles_m = (a.M + 127) / 128, tiles_n = (a.N + 64 * TN - 1) / (64 * TN);
  const int units = tiles_m * tiles_n * splits;
  int nb = device_cus();
  if (units < nb) nb = units;
  nb = (nb + 7) / 8 * 8;  // whole XCD rounds
  hipLaunchKernelGGL((gemm16_ksplit_kernel<TN, S, AK, BKC, EPI, TC, E>), dim3(nb), dim3(512), 0, s, a, units,
                     tiles_m, tiles_n, (const GemmGroupEntry*)nullptr);
}

// One launch of configuration cfg with the epilogue EPI and output type TC.
template <bool AK, bool BKC, int EPI, typename TC, typename E>
static void launch_cfg(int cfg, const GemmArgs& a, int splits, hipStream_t s) {
  if (cfg == kCfgKs192) launch_ksplit<3, 4, AK, BKC, EPI, TC, E>(a, splits, s);
  else if (cfg == kCfgKs128) launch_ksplit<2, 4, AK, BKC, EPI, TC, E>(a, splits, s);
  else if (cfg == kCfgPipe) launch_pipe<256, 256, 2, 4, 64, 2, 2, AK, BKC, EPI, TC, E>(a, splits, s);
  else if (cfg == kCfgPipe128) launch_pipe<128, 128, 2, 2, 64, 2, 2, AK, BKC, EPI, TC, E>(a, splits, s);
  else if (cfg == kCfgPipe192) {
    if constexpr (AK && BKC && EPI == EPI_STORE)
      launch_pipe<192, 128, 2, 2, 64, 2, 2, AK, BKC, EPI, TC, E>(a, splits, s);
    else
      launch_pipe<128, 128, 2, 2, 64, 2, 2, AK, BKC, EPI, TC, E>(a, splits, s);
  }
  else launch_small<128, 128, 2, 2, AK, BKC, EPI, TC, E>(a, splits, s);
}

template <bool AK, bool BKC, typename E>
static int dispatch_16(const GemmOp& op, const GemmArgs& a, int splits, hipStream_t s) {
  const int cfg = pick_cfg(op);
  if (splits > 1) {
    launch_cfg<AK, BKC, EPI_PARTIAL, float, E>(cfg, a, splits, s);
    return 0;
  }
  switch (op.epi) {
    case EPI_STORE:
      if (op.c_f32) launch_cfg<AK, BKC, EPI_STORE, float, E>(cfg, a, 1, s);
      else launch_cfg<AK, BKC, EPI_STORE, E, E>(cfg, a, 1, s);
      return 0;
    case EPI_RESID: launch_cfg<AK, BKC, EPI_RESID, float, E>(cfg, a, 1, s); return 0;
    case EPI_GELU: launch_cfg<AK, BKC, EPI_GELU, E, E>(cfg, a, 1, s); return 0;
    case EPI_DGELU: launch_cfg<AK, BKC, EPI_DGELU, E, E>(cfg, a, 1, s); return 0;
    default: return -1;
  }
}

// Split-K reduction of the 16-bit path (N and all leading dimensions are
// multiples of 8).
template <typename E>
static void launch_reduce16(const GemmOp& op, const GemmArgs& a, const float* part, int S, hipStream_t s) {
  const long ld = op.N;
  long total = (long)a.M_out * (op.N / 4);
  long blocks = (total + 255) / 256;
  if (blocks > 8192) blocks = 8192;
  dim3 g((unsigned)blocks), b(256);
  switch (op.epi) {
    case EPI_STORE:
      if (op.c_f32) hipLaunchKernelGGL((splitk_reduce4_kernel<EPI_STORE, float, E>), g, b, 0, s, a, part, S, ld);
      else hipLaunchKernelGGL((splitk_reduce4_kernel<EPI_STORE, E, E>), g, b, 0, s, a, part, S, ld);
      break;
    case EPI_RESID: hipLaunchKernelGGL((splitk_reduce4_kernel<EPI_RESID, float, E>), g, b, 0, s, a, part, S, ld); break;
    case EPI_GELU: hipLaunchKernelGGL((splitk_reduce4_kernel<EPI_GELU, E, E>), g, b, 0, s, a, part, S, ld); break;
    case EPI_DGELU: hipLaunchKernelGGL((splitk_reduce4_kernel<EPI_DGELU, E, E>), g, b, 0, s, a, part, S, ld); break;
    default: break;
  }
}

// Split-K reduction of the fp32 path.
static void launch_reduce32(const GemmOp& op, const GemmArgs& a, const float* part, int S, hipStream_t s) {
  const long ld = op.N;
  long total = (long)op.M * op.N;
  long blocks = (total + 255) / 256;
  if (blocks > 8192) blocks = 8192;
  dim3 g((unsigned)blocks), b(256);
  switch (op.epi) {
    case EPI_STORE: hipLaunchKernelGGL((splitk_reduce_kernel<EPI_STORE, float, float>), g, b, 0, s, a, part, S, ld); break;
    case EPI_RESID: hipLaunchKernelGGL((splitk_reduce_kernel<EPI_RESID, float, float>), g, b, 0, s, a, part, S, ld); break;
    case EPI_GELU: hipLaunchKernelGGL((splitk_reduce_kernel<EPI_GELU, float, float>), g, b, 0, s, a, part, S, ld); break;
    case EPI_DGELU: hipLaunchKernelGGL((splitk_reduce_kernel<EPI_DGELU, float, float>), g, b, 0, s, a, part, S, ld); break;
    default: break;
  }
}

// fp32 path: 64 x 64 tiles; split K while the tiles leave CUs idle
// K slices of the fp32 kernel: its tiles are serial K loops on one CU each,
// and the small fp32 shapes have few of them (10-12 tiles of 64 x 64 for the
// 128-wide model at 320 tokens), so K is split until the slices fill the CUs
// or a slice would hold fewer than 64 K-values; the partials are summed in
// slice order by the reduction pass.
static int gemm32_splits(const GemmOp& op) {
  if (op.force_split > 0) return op.force_split;
  const long tiles = (long)((op.M + 63) / 64) * ((op.N + 63) / 64);
  int splits = 1;
  while (tiles * splits < 256 && op.K / (splits * 2) >= 64) splits *= 2;
  return splits;
}

long gemm_ws_floats_needed(const GemmOp& op, bool h16) {
  if (op.M <= 0 || op.N <= 0 || op.K <= 0) return 0;
  const int splits = h16 ? gemm16_splits(op) : gemm32_splits(op);
  return splits > 1 ? (long)splits * op.M * op.N : 0;
}

int gemm_check(const GemmOp& op, bool h16) {
  if (op.cfg > 0 && (!h16 || !cfg_allowed(op, op.cfg))) return -1;
  if (!h16) return op.colsum ? -1 : 0;
  if (op.M <= 0 || op.N <= 0) return 0;
  if (!check_16(op)) return -1;
  if (op.colsum && gemm16_colsum_rows(op) == 0) return -1;
  return 0;
}

template <typename E>
static int gemm16(const GemmOp& op, float* ws, long ws_floats, hipStream_t s) {
  if (gemm_check(op, true)) return -1;
  if (op.M <= 0 || op.N <= 0) return 0;
  GemmArgs a = make_args(op);
  int splits = gemm16_splits(op);
  if (splits > 1 && (long)splits * op.M * op.N > ws_floats) splits = 1;
  // K slices are multiples of the K step (which can leave a single slice)
  int per = op.K;
  if (splits > 1) {
    per = (op.K + splits - 1) / splits;
    per = (per + kBK - 1) / kBK * kBK;
    splits = (op.K + per - 1) / per;
  }
  GemmArgs pa = a;
  if (splits > 1) {
    pa.C = ws;
    pa.ldc = op.N;
    pa.k_split = per;
    pa.split_stride = (long)op.M * op.N;
  }
  int rc;
  if (op.a_kc && op.b_kc) rc = dispatch_16<true, true, E>(op, pa, splits, s);
  else if (op.a_kc) rc = dispatch_16<true, false, E>(op, pa, splits, s);
  else if (!op.b_kc) rc = dispatch_16<false, false, E>(op, pa, splits, s);
  else rc = dispatch_16<false, true, E>(op, pa, splits, s);
  if (rc) return rc;
  if (splits > 1) launch_reduce16<E>(op, a, ws, splits, s);
  return 0;
}

int gemm_bf16(const GemmOp& op, float* ws, long ws_floats, hipStream_t s) { return gemm16<bf16>(op, ws, ws_floats, s); }
int gemm_f16(const GemmOp& op, float* ws, long ws_floats, hipStream_t s) { return gemm16<f16>(op, ws, ws_floats, s); }

// ------------------------------------------------------- grouped launch
// Weight gradients (both operands M/N-contiguous, fp32 output, plain store,
// no bias) of many GEMMs in one persistent launch of the K-split kernel, one
// whole tile over all of K per unit: no K slices, so no partial sums and no
// reduction pass, and one launch's fixed cost (first loads, last stores)
// instead of one per GEMM.
long gemm_group_table_bytes(int n) { return (long)(n + 1) * (long)sizeof(GemmGroupEntry); }

int gemm_group_plan(const GemmOp* ops, int n, void* table, int* tn, float* const* part) {
  if (n < 1 || !table || !tn) return -1;
  for (int i = 0; i < n; ++i) {
    const GemmOp& op = ops[i];
    // K slices (force_split > 1) need their partial-sum buffer
    const bool sliced = op.force_split > 1 && part && part[i];
    if (op.a_kc || op.b_kc || op.epi != EPI_STORE || !op.c_f32 || op.bias || op.R || op.aux || op.colsum ||
        op.cfg != 0 || (op.force_split > 1 && !sliced) || op.M <= 0 || op.N <= 0 || op.K <= 0 || !check_16(op))
      return -1;
  }
  // 128 x 192 tiles, also where a width is not a multiple of 192 (the last
  // tile column is then partly empty): on the 512- and 2048-wide weight
  // gradients of a d_model 512 model they measured 1.6% faster than 128 x 128
  // tiles, whose 1.4 times as many units take more rounds of the CUs
  *tn = 3;
  const int bn = 64 * *tn;
  GemmGroupEntry* e = static_cast<GemmGroupEntry*>(table);
  long units = 0;
  // (field by field into zeroed entries: the table's bytes, padding
  // included, depend only on the ops, so callers can compare tables bytewise)
  std::memset(table, 0, (size_t)gemm_group_table_bytes(n));
  for (int i = 0; i < n; ++i) {
    const GemmArgs a = make_args(ops[i]);
    GemmArgs& d = e[i].a;
    d.A = a.A; d.lda = a.lda; d.B = a.B; d.ldb = a.ldb; d.C = a.C; d.ldc = a.ldc;
    d.bias = a.bias; d.R = a.R; d.ldr = a.ldr; d.aux = a.aux; d.ld_aux = a.ld_aux;
    d.M = a.M; d.N = a.N; d.K = a.K; d.M_out = a.M_out; d.k_split = a.k_split;
    d.split_stride = a.split_stride; d.colsum = a.colsum;
    int slices = 1;
    if (ops[i].force_split > 1) {
      // whole K steps of 64 per slice; slice z of tile (m, n) stores into
      // part[i] + z * M * N, rows of N floats
      const int per = ((ops[i].K + ops[i].force_split - 1) / ops[i].force_split + 63) / 64 * 64;
      slices = (ops[i].K + per - 1) / per;
      d.C = part[i]; d.ldc = ops[i].N; d.k_split = per; d.split_stride = (long)ops[i].M * ops[i].N;
    }
    e[i].first_unit = (int)units;
    e[i].tiles_m = (ops[i].M + 127) / 128;
    e[i].tiles_n = (ops[i].N + bn - 1) / bn;
    units += (long)e[i].tiles_m * e[i].tiles_n * slices;
    if (units > (1L << 30)) return -1;
  }
  e[n].first_unit = (int)units;
  return (int)units;
}

// (the partial-sum epilogue of a single slice is the plain fp32 store
// without bias, and it keeps the K loop's registers those of the split-K
// weight-gradient launches)
template <int TN, typename E>
static void launch_group(const void* table, int units, hipStream_t s) {
  int nb = device_cus();
  if (units < nb) nb = units;
  nb = (nb + 7) / 8 * 8;  // whole XCD rounds
  hipLaunchKernelGGL((gemm16_ksplit_kernel<TN, 4, false, false, EPI_PARTIAL, float, E, true>), dim3(nb), dim3(512),
                     0, s, GemmArgs{}, units, 0, 0, static_cast<const GemmGroupEntry*>(table));
}

int gemm_group_slices_of(const GemmOp& op) {
  if (op.force_split <= 1) return 1;
  const int per = ((op.K + op.force_split - 1) / op.force_split + 63) / 64 * 64;
  return (op.K + per - 1) / per;
}

// dst[r][c] = sum over z < S of part[z][r][c] in slice order (rows r <
// rows, 4 columns per thread), for the sliced GEMMs of a grouped launch
__global__ void __launch_bounds__(256) group_reduce_kernel(GroupReduce gr) {
  const int e = blockIdx.y;
  const float* __restrict__ part = gr.part[e];
  float* __restrict__ dst = gr.dst[e];
  const int nq = gr.cols[e] >> 2;
  const long total = (long)gr.rows[e] * nq, stride4 = gr.stride[e] / 4;
  for (long q = (long)blockIdx.x * 256 + threadIdx.x; q < total; q += (long)gridDim.x * 256) {
    const long row = q / nq, col = (q - row * nq) * 4;
    const f32x4_t* src = reinterpret_cast<const f32x4_t*>(part + row * gr.cols[e] + col);
    f32x4_t acc = __builtin_nontemporal_load(src);
    for (int z = 1; z < gr.S[e]; ++z) acc += __builtin_nontemporal_load(src + z * stride4);
    *reinterpret_cast<f32x4_t*>(dst + row * gr.ldc[e] + col) = acc;
  }
}

void launch_group_reduce(const GroupReduce& gr, hipStream_t s) {
  if (gr.n <= 0) return;
  long most = 0;
  for (int i = 0; i < gr.n; ++i) most = std::max(most, (long)gr.rows[i] * (gr.cols[i] >> 2));
  const unsigned bx = (unsigned)std::min(1024L, (most + 255) / 256);
  hipLaunchKernelGGL(group_reduce_kernel, dim3(bx, gr.n), dim3(256), 0, s, gr);
}

int gemm_group_launch(bool f16_ops, int tn, const void* table_dev, int units, hipStream_t s) {
  if (!table_dev || units < 0 || tn != 3) return -1;
  if (units == 0) return 0;
  if (f16_ops) launch_group<3, f16>(table_dev, units, s);
  else launch_group<3, bf16>(table_dev, units, s);
  return 0;
}

int gemm_cus() { return device_cus(); }

template <bool AK, bool BKC>
static int dispatch_f32(const GemmOp& op, const GemmArgs& a, int splits, hipStream_t s) {
  dim3 grid((a.N + 63) / 64, (a.M + 63) / 64, splits), b(256);
  int epi = splits > 1 ? EPI_PARTIAL : op.epi;
  switch (epi) {
    case EPI_PARTIAL: hipLaunchKernelGGL((gemm_f32_kernel<AK, BKC, EPI_PARTIAL>), grid, b, 0, s, a); return 0;
    case EPI_STORE: hipLaunchKernelGGL((gemm_f32_kernel<AK, BKC, EPI_STORE>), grid, b, 0, s, a); return 0;
    case EPI_RESID: hipLaunchKernelGGL((gemm_f32_kernel<AK, BKC, EPI_RESID>), grid, b, 0, s, a); return 0;
    case EPI_GELU: hipLaunchKernelGGL((gemm_f32_kernel<AK, BKC, EPI_GELU>), grid, b, 0, s, a); return 0;
    case EPI_DGELU: hipLaunchKernelGGL((gemm_f32_kernel<AK, BKC, EPI_DGELU>), grid, b, 0, s, a); return 0;
    default: return -1;
  }
}

int gemm_f32(const GemmOp& op, float* ws, long ws_floats, hipStream_t s) {
  if (gemm_check(op, false)) return -1;  // (colsum: 16-bit GELU' epilogue only)
  if (op.M <= 0 || op.N <= 0) return 0;
  GemmArgs a = make_args(op);
  int splits = gemm32_splits(op);
  if (splits > 1 && (long)splits * op.M * op.N > ws_floats) splits = 1;
  // K slices are multiples of 16 (which can leave a single slice)
  int per = op.K;
  if (splits > 1) {
    per = (op.K + splits - 1) / splits;
    per = (per + 15) / 16 * 16;
    splits = (op.K + per - 1) / per;
  }
  if (splits > 1) {
    GemmArgs pa = a;
    pa.C = ws;
    pa.ldc = op.N;
    pa.k_split = per;
    pa.split_stride = (long)op.M * op.N;
    int rc;
    if (op.a_kc && op.b_kc) rc = dispatch_f32<true, true>(op, pa, splits, s);
    else if (op.a_kc) rc = dispatch_f32<true, false>(op, pa, splits, s);
    else if (!op.b_kc) rc = dispatch_f32<false, false>(op, pa, splits, s);
    else rc = dispatch_f32<false, true>(op, pa, splits, s);
    if (rc) return rc;
    launch_reduce32(op, a, ws, splits, s);
    return 0;
  }
  if (op.a_kc && op.b_kc) return dispatch_f32<true, true>(op, a, 1, s);
  if (op.a_kc) return dispatch_f32<true, false>(op, a, 1, s);
  if (!op.b_kc) return dispatch_f32<false, false>(op, a, 1, s);
  return dispatch_f32<false, true>(op, a, 1, s);
}

}  // namespace lm
