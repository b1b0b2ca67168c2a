// Dense contractions of the step: the QKV, attention-output, MLP and tied
// vocabulary projections, forward and backward (Y = X W^T, dX = dY W,
// dW = dY^T X), with fused epilogues (bias, GELU, its derivative, residual
// add). Matrix multiplication is where the time goes (Feste page, "Tensor
// Operations": matmul is the bottleneck); its CPU tiling for L1 is prior art,
// here the contraction runs on the gfx950 matrix cores.
//
// bf16 path: 256 threads (2 x 2 wavefronts), block tile BM x BN, K step 64,
// two LDS stages (global loads for step k+1 are in flight while step k runs on
// the MFMA units). LDS rows hold 64 K-values plus 8 bf16 of padding (144 B),
// which keeps the 16-byte fragment reads of 32 consecutive rows conflict-free.
// Operands whose contiguous axis is M or N (the backward's dY^T and X^T, and
// W read along its rows for dX) are loaded as 8 x 8 bf16 blocks and transposed
// in registers before the LDS store, so every fragment read is K-contiguous.
// Each wavefront computes (BM/2) x (BN/2) with v_mfma_f32_32x32x16_bf16.
//
// fp32 path: fp32 matrix and vector peaks are equal on this chip (157 TF), so
// the fp32 GEMM is a plain LDS-tiled FMA kernel (64 x 64 tile, 4 x 4 per
// thread).
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
    float u = acc + (p.bias ? p.bias[col] : 0.f);
    Act<TA>::st(reinterpret_cast<TA*>(p.C), row * p.ldc + col, u);
    Act<TA>::st(reinterpret_cast<TA*>(p.aux), row * p.ld_aux + col, gelu_f(u));
  } else if (EPI == EPI_DGELU) {
    float u = Act<TA>::ld(reinterpret_cast<const TA*>(p.aux), row * p.ld_aux + col);
    Act<TA>::st(reinterpret_cast<TA*>(p.C), row * p.ldc + col, acc * gelu_grad_f(u));
  }
}

// ------------------------------------------------------------ bf16 MFMA GEMM
constexpr int kBK = 64;
constexpr int kPitch = 72;  // bf16 per LDS row (64 + 8 padding)

__device__ __forceinline__ uint32_t word_of(const uint4& v, int q) {
  return q == 0 ? v.x : q == 1 ? v.y : q == 2 ? v.z : v.w;
}

// Loads the ROWS x 64 tile of one operand for the K step at k0 into registers.
// K-contiguous: ROWS * 8 chunks of 8 bf16. Otherwise: ROWS 8 x 8 blocks.
template <int ROWS, bool KC>
struct TileLoader {
  static constexpr int NCH = KC ? (ROWS * 8 + 255) / 256 : 1;  // K-contiguous chunks per thread
  static constexpr int NBLK = KC ? 0 : (ROWS + 255) / 256;     // 8x8 blocks per thread (<= 1 here)
  uint4 r[KC ? NCH : 8];
  static_assert(KC || ROWS <= 256, "one 8x8 block per thread at most");

  __device__ __forceinline__ void load(const bf16* __restrict__ base, long ld, int row0, int rows_total, int k0,
                                       int k_end, int tid) {
    if (KC) {
#pragma unroll
      for (int i = 0; i < NCH; ++i) {
        int c = tid + i * 256;
        int row = c >> 3, kc = c & 7;
        int gr = row0 + row, gk = k0 + kc * 8;
        if (c < ROWS * 8 && gr < rows_total && gk < k_end)
          r[i] = *reinterpret_cast<const uint4*>(base + (long)gr * ld + gk);
        else
          r[i] = make_uint4(0, 0, 0, 0);
      }
    } else {
      int b = tid;
      if (b < ROWS) {
        int ib = b % (ROWS / 8), kb = b / (ROWS / 8);
        int gi = row0 + ib * 8;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          int gk = k0 + kb * 8 + j;
          if (gi < rows_total && gk < k_end)
            r[j] = *reinterpret_cast<const uint4*>(base + (long)gk * ld + gi);
          else
            r[j] = make_uint4(0, 0, 0, 0);
        }
      }
    }
  }

  __device__ __forceinline__ void store(bf16* __restrict__ s, int tid) const {
    if (KC) {
#pragma unroll
      for (int i = 0; i < NCH; ++i) {
        int c = tid + i * 256;
        if (c < ROWS * 8) {
          int row = c >> 3, kc = c & 7;
          *reinterpret_cast<uint4*>(s + row * kPitch + kc * 8) = r[i];
        }
      }
    } else {
      int b = tid;
      if (b < ROWS) {
        int ib = b % (ROWS / 8), kb = b / (ROWS / 8);
        // r[j] holds 8 consecutive rows-of-the-tile (i) at k = kb*8 + j.
        // Output row i = ib*8 + c gets the 8 k-values of element c.
#pragma unroll
        for (int c = 0; c < 8; ++c) {
          uint32_t o[4];
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            uint32_t lo = word_of(r[2 * j], c >> 1), hi = word_of(r[2 * j + 1], c >> 1);
            o[j] = (c & 1) ? ((lo >> 16) | (hi & 0xffff0000u)) : ((lo & 0xffffu) | (hi << 16));
          }
          *reinterpret_cast<uint4*>(s + (ib * 8 + c) * kPitch + kb * 8) = make_uint4(o[0], o[1], o[2], o[3]);
        }
      }
    }
  }
};

template <int BM, int BN, bool AK, bool BKC, int EPI, typename TC>
__global__ void __launch_bounds__(256) gemm_bf16_kernel(GemmArgs p) {
  constexpr int WM = BM / 2, WN = BN / 2;
  constexpr int TM = WM / 32, TN = WN / 32;
  __shared__ __attribute__((aligned(16))) bf16 sA[2][BM * kPitch];
  __shared__ __attribute__((aligned(16))) bf16 sB[2][BN * kPitch];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int m0 = blockIdx.y * BM, n0 = blockIdx.x * BN;
  const int z = blockIdx.z;
  const int k_begin = z * p.k_split;
  const int k_end = min(p.K, k_begin + p.k_split);
  const int nk = (k_end - k_begin + kBK - 1) / kBK;
  const bf16* A = reinterpret_cast<const bf16*>(p.A);
  const bf16* B = reinterpret_cast<const bf16*>(p.B);

  TileLoader<BM, AK> la;
  TileLoader<BN, BKC> lb;
  f32x16_t acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;

  if (nk > 0) {
    la.load(A, p.lda, m0, p.M, k_begin, k_end, tid);
    lb.load(B, p.ldb, n0, p.N, k_begin, k_end, tid);
    la.store(sA[0], tid);
    lb.store(sB[0], tid);
  }
  __syncthreads();

  for (int it = 0; it < nk; ++it) {
    const int cur = it & 1;
    if (it + 1 < nk) {
      la.load(A, p.lda, m0, p.M, k_begin + (it + 1) * kBK, k_end, tid);
      lb.load(B, p.ldb, n0, p.N, k_begin + (it + 1) * kBK, k_end, tid);
    }
    const bf16* a_s = sA[cur];
    const bf16* b_s = sB[cur];
#pragma unroll
    for (int ks = 0; ks < kBK / 16; ++ks) {
      bf16x8_t af[TM], bfr[TN];
      const int kof = ks * 16 + (lane >> 5) * 8;
#pragma unroll
      for (int i = 0; i < TM; ++i)
        af[i] = *reinterpret_cast<const bf16x8_t*>(a_s + (wm * WM + i * 32 + (lane & 31)) * kPitch + kof);
#pragma unroll
      for (int j = 0; j < TN; ++j)
        bfr[j] = *reinterpret_cast<const bf16x8_t*>(b_s + (wn * WN + j * 32 + (lane & 31)) * kPitch + kof);
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bfr[j], acc[i][j], 0, 0, 0);
    }
    if (it + 1 < nk) {
      la.store(sA[cur ^ 1], tid);
      lb.store(sB[cur ^ 1], tid);
    }
    __syncthreads();
  }

  // accumulator element e of tile (i, j): row (e/4)*8 + (lane/32)*4 + e%4, column lane%32
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j) {
      const long col = n0 + wn * WN + j * 32 + (lane & 31);
      if (col >= p.N) continue;
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const long row = m0 + wm * WM + i * 32 + (e >> 2) * 8 + (lane >> 5) * 4 + (e & 3);
        if (row < p.M_out) epilogue<EPI, TC, bf16>(p, row, col, acc[i][j][e], z);
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

// ------------------------------------------------------------- dispatch
static GemmArgs make_args(const GemmOp& op) {
  GemmArgs a;
  a.A = op.A; a.lda = op.lda; a.B = op.B; a.ldb = op.ldb; a.C = op.C; a.ldc = op.ldc;
  a.bias = op.bias; a.R = op.R; a.ldr = op.ldr; a.aux = op.aux; a.ld_aux = op.ld_aux;
  a.M = op.M; a.N = op.N; a.K = op.K; a.k_split = op.K; a.split_stride = 0;
  a.M_out = op.M_out > 0 && op.M_out < op.M ? op.M_out : op.M;
  return a;
}

static bool check_bf16(const GemmOp& op) {
  if (op.lda % 8 || op.ldb % 8) return false;
  if ((op.a_kc || op.b_kc) && op.K % 8) return false;
  if (!op.a_kc && op.M % 8) return false;
  if (!op.b_kc && op.N % 8) return false;
  if (!op.a_kc && !op.b_kc) return true;
  return true;
}

static void tile_for(const GemmOp& op, int& BM, int& BN) {
  BM = 128;
  BN = 128;
  (void)op;
}

int gemm_bf16_splits(const GemmOp& op) {
  if (op.force_split > 0) return op.force_split;
  int BM, BN;
  tile_for(op, BM, BN);
  long tiles = (long)((op.M + BM - 1) / BM) * ((op.N + BN - 1) / BN);
  // split K when the tile grid cannot fill the 256 compute units and K is long
  int s = 1;
  while (tiles * s < 256 && op.K / (s * 2) >= 512) s *= 2;
  return s;
}

template <int BM, int BN, bool AK, bool BKC, int EPI, typename TC>
static void launch_bf16(const GemmArgs& a, int splits, hipStream_t s) {
  dim3 grid((a.N + BN - 1) / BN, (a.M + BM - 1) / BM, splits);
  hipLaunchKernelGGL((gemm_bf16_kernel<BM, BN, AK, BKC, EPI, TC>), grid, dim3(256), 0, s, a);
}

template <bool AK, bool BKC>
static int dispatch_bf16_epi(const GemmOp& op, const GemmArgs& a, int splits, hipStream_t s) {
  if (splits > 1) {
    launch_bf16<128, 128, AK, BKC, EPI_PARTIAL, float>(a, splits, s);
    return 0;
  }
  switch (op.epi) {
    case EPI_STORE:
      if (op.c_f32) launch_bf16<128, 128, AK, BKC, EPI_STORE, float>(a, 1, s);
      else launch_bf16<128, 128, AK, BKC, EPI_STORE, bf16>(a, 1, s);
      return 0;
    case EPI_RESID: launch_bf16<128, 128, AK, BKC, EPI_RESID, float>(a, 1, s); return 0;
    case EPI_GELU: launch_bf16<128, 128, AK, BKC, EPI_GELU, bf16>(a, 1, s); return 0;
    case EPI_DGELU: launch_bf16<128, 128, AK, BKC, EPI_DGELU, bf16>(a, 1, s); return 0;
    default: return -1;
  }
}

template <typename TA>
static void launch_reduce(const GemmOp& op, const GemmArgs& a, const float* part, int S, hipStream_t s) {
  long total = (long)op.M * op.N;
  long blocks = (total + 255) / 256;
  if (blocks > 8192) blocks = 8192;
  dim3 g((unsigned)blocks), b(256);
  long ld = op.N;
  switch (op.epi) {
    case EPI_STORE:
      if (op.c_f32) hipLaunchKernelGGL((splitk_reduce_kernel<EPI_STORE, float, TA>), g, b, 0, s, a, part, S, ld);
      else hipLaunchKernelGGL((splitk_reduce_kernel<EPI_STORE, TA, TA>), g, b, 0, s, a, part, S, ld);
      break;
    case EPI_RESID: hipLaunchKernelGGL((splitk_reduce_kernel<EPI_RESID, float, TA>), g, b, 0, s, a, part, S, ld); break;
    case EPI_GELU: hipLaunchKernelGGL((splitk_reduce_kernel<EPI_GELU, TA, TA>), g, b, 0, s, a, part, S, ld); break;
    case EPI_DGELU: hipLaunchKernelGGL((splitk_reduce_kernel<EPI_DGELU, TA, TA>), g, b, 0, s, a, part, S, ld); break;
    default: break;
  }
}

int gemm_bf16(const GemmOp& op, float* ws, long ws_floats, hipStream_t s) {
  if (op.M <= 0 || op.N <= 0) return 0;
  if (!check_bf16(op)) return -1;
  GemmArgs a = make_args(op);
  int splits = gemm_bf16_splits(op);
  if (splits > 1 && (long)splits * op.M * op.N > ws_floats) splits = 1;
  if (splits > 1) {
    // K slices are multiples of the K step
    int per = (op.K + splits - 1) / splits;
    per = (per + kBK - 1) / kBK * kBK;
    splits = (op.K + per - 1) / per;
    GemmArgs pa = a;
    pa.C = ws;
    pa.ldc = op.N;
    pa.k_split = per;
    pa.split_stride = (long)op.M * op.N;
    int rc;
    if (op.a_kc && op.b_kc) rc = dispatch_bf16_epi<true, true>(op, pa, splits, s);
    else if (op.a_kc) rc = dispatch_bf16_epi<true, false>(op, pa, splits, s);
    else if (!op.b_kc) rc = dispatch_bf16_epi<false, false>(op, pa, splits, s);
    else rc = dispatch_bf16_epi<false, true>(op, pa, splits, s);
    if (rc) return rc;
    launch_reduce<bf16>(op, a, ws, splits, s);
    return 0;
  }
  if (op.a_kc && op.b_kc) return dispatch_bf16_epi<true, true>(op, a, 1, s);
  if (op.a_kc) return dispatch_bf16_epi<true, false>(op, a, 1, s);
  if (!op.b_kc) return dispatch_bf16_epi<false, false>(op, a, 1, s);
  return dispatch_bf16_epi<false, true>(op, a, 1, s);
}

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
  if (op.M <= 0 || op.N <= 0) return 0;
  GemmArgs a = make_args(op);
  long tiles = (long)((op.M + 63) / 64) * ((op.N + 63) / 64);
  int splits = op.force_split > 0 ? op.force_split : 1;
  if (op.force_split <= 0)
    while (tiles * splits < 256 && op.K / (splits * 2) >= 256) splits *= 2;
  if (splits > 1 && (long)splits * op.M * op.N > ws_floats) splits = 1;
  if (splits > 1) {
    int per = (op.K + splits - 1) / splits;
    per = (per + 15) / 16 * 16;
    splits = (op.K + per - 1) / per;
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
    launch_reduce<float>(op, a, ws, splits, s);
    return 0;
  }
  if (op.a_kc && op.b_kc) return dispatch_f32<true, true>(op, a, 1, s);
  if (op.a_kc) return dispatch_f32<true, false>(op, a, 1, s);
  if (!op.b_kc) return dispatch_f32<false, false>(op, a, 1, s);
  return dispatch_f32<false, true>(op, a, 1, s);
}

}  // namespace lm
