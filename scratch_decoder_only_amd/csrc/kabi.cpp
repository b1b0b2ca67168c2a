// Per-kernel C entry points (the kernels of the step, one at a time).
#include <hip/hip_runtime.h>

#include <cmath>
#include <mutex>
#include <type_traits>
#include <vector>

#include "../../include/lmstep_kernels.h"
#include "kernels.h"

using namespace lm;

static hipStream_t S(void* s) { return reinterpret_cast<hipStream_t>(s); }

// precision: 0 fp32, 1 bf16, 2 fp16 (the activation / operand storage type);
// f gets a null pointer of that type as a tag. Other values: -1.
template <typename F>
static int with_prec(int precision, F&& f) {
  switch (precision) {
    case 0: return f(static_cast<float*>(nullptr));
    case 1: return f(static_cast<bf16*>(nullptr));
    case 2: return f(static_cast<f16*>(nullptr));
    default: return -1;
  }
}
#define ACT_T std::remove_pointer_t<decltype(tag)>

extern "C" {

int lmk_gemm_cfg(int cfg, int precision, int M, int N, int K, const void* A, int64_t lda, int a_kc, const void* B,
                 int64_t ldb, int b_kc, void* C, int64_t ldc, int epi, int c_f32, const float* bias, const float* R,
                 int64_t ldr, void* aux, int64_t ld_aux, int force_split, int M_out, float* ws, int64_t ws_floats,
                 void* stream) {
  if (!A || !B || !C || M < 0 || N < 0 || K < 0 || epi < 0 || epi > 3 || cfg < 0) return -1;
  GemmOp op;
  op.cfg = cfg;
  op.M = M; op.N = N; op.K = K;
  op.A = A; op.lda = lda; op.a_kc = a_kc != 0;
  op.B = B; op.ldb = ldb; op.b_kc = b_kc != 0;
  op.C = C; op.ldc = ldc; op.epi = epi; op.c_f32 = c_f32 != 0;
  op.bias = bias; op.R = R; op.ldr = ldr; op.aux = aux; op.ld_aux = ld_aux;
  op.force_split = force_split; op.M_out = M_out;
  if (epi == EPI_RESID && !R) return -1;
  if ((epi == EPI_GELU || epi == EPI_DGELU) && !aux) return -1;
  if (precision == 2) return gemm_f16(op, ws, ws_floats, S(stream));
  if (precision == 1) return gemm_bf16(op, ws, ws_floats, S(stream));
  if (precision == 0) return gemm_f32(op, ws, ws_floats, S(stream));
  return -1;
}

int lmk_gemm(int precision, int M, int N, int K, const void* A, int64_t lda, int a_kc, const void* B, int64_t ldb,
             int b_kc, void* C, int64_t ldc, int epi, int c_f32, const float* bias, const float* R, int64_t ldr,
             void* aux, int64_t ld_aux, int force_split, int M_out, float* ws, int64_t ws_floats, void* stream) {
  return lmk_gemm_cfg(0, precision, M, N, K, A, lda, a_kc, B, ldb, b_kc, C, ldc, epi, c_f32, bias, R, ldr, aux,
                      ld_aux, force_split, M_out, ws, ws_floats, stream);
}

int64_t lmk_gemm_group_table_bytes(int n) { return n < 1 ? -1 : gemm_group_table_bytes(n); }

int lmk_gemm_group(int precision, int n, const int* mnk, const void* const* A, const int64_t* lda,
                   const void* const* B, const int64_t* ldb, float* const* C, const int64_t* ldc, void* table,
                   int64_t table_bytes, void* stream) {
  if ((precision != 1 && precision != 2) || n < 1 || !mnk || !A || !lda || !B || !ldb || !C || !ldc || !table)
    return -1;
  if (table_bytes < gemm_group_table_bytes(n)) return -1;
  std::vector<GemmOp> ops(n);
  for (int i = 0; i < n; ++i) {
    if (!A[i] || !B[i] || !C[i]) return -1;
    GemmOp& op = ops[i];
    op.M = mnk[3 * i]; op.N = mnk[3 * i + 1]; op.K = mnk[3 * i + 2];
    op.A = A[i]; op.lda = lda[i]; op.a_kc = false;
    op.B = B[i]; op.ldb = ldb[i]; op.b_kc = false;
    op.C = C[i]; op.ldc = ldc[i]; op.epi = EPI_STORE; op.c_f32 = true;
  }
  std::vector<char> host(gemm_group_table_bytes(n));
  int tn = 0;
  const int units = gemm_group_plan(ops.data(), n, host.data(), &tn);
  if (units < 0) return -1;
  hipStream_t s = S(stream);
  if (hipStreamSynchronize(s) != hipSuccess ||
      hipMemcpy(table, host.data(), host.size(), hipMemcpyHostToDevice) != hipSuccess)
    return -1;
  return gemm_group_launch(precision == 2, tn, table, units, s);
}

static bool ln_shape_ok(int M, int C) { return M >= 0 && C >= 128 && C <= 1024 && C % 128 == 0; }

int lmk_layernorm_fwd(int precision, const float* x, const float* g, const float* b, int M, int C, float eps, void* y,
                      float* mu, float* rstd, void* stream) {
  if (!ln_shape_ok(M, C)) return -1;
  return with_prec(precision, [&](auto tag) {
    launch_ln_fwd<ACT_T>(x, g, b, M, C, eps, reinterpret_cast<ACT_T*>(y), mu, rstd, S(stream));
    return 0;
  });
}

int64_t lmk_layernorm_bwd_ws_floats(int M, int C) {
  return 3L * ((M + kLnRowsPerBlock - 1) / kLnRowsPerBlock) * C;
}

int lmk_layernorm_bwd(int precision, const float* dy, const float* x, const float* mu, const float* rstd,
                      const float* g, int M, int C, const float* g_in, float* g_out, void* g_act, float* dgamma,
                      float* dbeta, float* dsum, float* ws, void* stream) {
  if (!ln_shape_ok(M, C) || M == 0) return -1;
  long nb = (M + kLnRowsPerBlock - 1) / kLnRowsPerBlock;
  float* pc = dsum ? ws + 2 * nb * C : nullptr;
  const int rc = with_prec(precision, [&](auto tag) {
    launch_ln_bwd<ACT_T>(dy, x, mu, rstd, g, M, C, g_in, g_out, reinterpret_cast<ACT_T*>(g_act), ws, ws + nb * C,
                         pc, S(stream));
    return 0;
  });
  if (rc) return rc;
  launch_colsum_partials(ws, ws + nb * C, (int)nb, C, dgamma, dbeta, S(stream), pc, dsum);
  return 0;
}

int64_t lmk_colsum_ws_floats(int M, int N) { return (int64_t)((M + kColRows - 1) / kColRows) * N; }

int lmk_colsum(int precision_of_a, const void* a, int64_t lda, int M, int N, float* out, float* ws, void* stream) {
  if (M <= 0 || N <= 0 || N % 4 || lda % 4) return -1;
  return with_prec(precision_of_a, [&](auto tag) {
    launch_colsum<ACT_T>(reinterpret_cast<const ACT_T*>(a), lda, M, N, ws, out, S(stream));
    return 0;
  });
}

int lmk_index_layout(const int32_t* doc, int B, int T, int32_t* start, int32_t* end, int32_t* pos, uint32_t* flags,
                     void* stream) {
  if (B <= 0 || T <= 0) return -1;
  launch_index_layout(doc, B, T, start, end, pos, flags, S(stream));
  return 0;
}

int lmk_embed_fwd(const int32_t* tok, const int32_t* pos, const float* wte, const float* wpe, int M, int C, int V,
                  float* x, uint32_t* flags, void* stream) {
  if (M <= 0 || C % 2) return -1;
  launch_embed_fwd(tok, pos, wte, wpe, M, C, V, x, flags, S(stream));
  return 0;
}

int lmk_attn_fwd(int precision, const void* qkv, const int32_t* start, const int32_t* end, int B, int T, int H, int D,
                 void* o, float* lse, void* stream) {
  if (B <= 0 || T <= 0 || H <= 0 || (D != 32 && D != 64)) return -1;
  AttnArgs a{};
  a.qkv = qkv; a.start = start; a.end = end; a.B = B; a.T = T; a.H = H; a.D = D; a.o = o; a.lse = lse;
  return with_prec(precision, [&](auto tag) {
    if constexpr (std::is_same_v<ACT_T, float>) return attn_fwd_f32(a, S(stream));
    else return attn_fwd16<ACT_T>(a, S(stream));
  });
}

int lmk_attn_bwd(int precision, const void* qkv, const void* o, const float* lse, const void* dout,
                 const int32_t* start, const int32_t* end, int B, int T, int H, int D, float* delta, void* dqkv,
                 void* stream) {
  if (B <= 0 || T <= 0 || H <= 0 || (D != 32 && D != 64)) return -1;
  AttnArgs a{};
  a.qkv = qkv; a.start = start; a.end = end; a.B = B; a.T = T; a.H = H; a.D = D;
  a.o = const_cast<void*>(o); a.lse = const_cast<float*>(lse); a.dout = dout; a.delta = delta; a.dqkv = dqkv;
  return with_prec(precision, [&](auto tag) {
    if constexpr (std::is_same_v<ACT_T, float>) return attn_bwd_f32(a, S(stream));
    else return attn_bwd16<ACT_T>(a, S(stream));
  });
}

int lmk_xent(int precision, void* z, int64_t ldz, int M, int V, const int32_t* tgt, float* loss, int32_t* ws_n,
             float* ws_rows, uint32_t* flags, const float* loss_scale, void* stream) {
  if (M <= 0 || V <= 0 || ldz < V || ldz % 8 || precision < 0 || precision > 2) return -1;
  launch_count_valid(tgt, M, V, ws_n, loss, flags, S(stream));
  with_prec(precision, [&](auto tag) {
    launch_xent<ACT_T>(reinterpret_cast<ACT_T*>(z), ldz, M, V, tgt, ws_n, ws_rows, loss_scale, S(stream));
    return 0;
  });
  launch_loss_reduce(ws_rows, M, ws_n, loss, S(stream));
  return 0;
}

// Scratch of lmk_xent_noalloc: the valid-target count (int32, first 256
// bytes) and one loss per row, in device memory the library reserves once per
// GPU. The name is a host-side stand-in for the device array: host code uses
// only the address hipGetSymbolAddress returns for the current device.
constexpr int kXentNoallocRows = 1 << 16;
constexpr int kXentNoallocHead = 64;  // floats before the per-row losses
static __device__ __align__(256) float scratch[kXentNoallocHead + kXentNoallocRows];

// The address of this GPU's scratch, looked up once per device (with that
// device current) and kept; null if the lookup fails.
static float* xent_scratch() {
  static std::mutex mu;
  static float* ptr[64] = {nullptr};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return nullptr;
  std::lock_guard<std::mutex> lock(mu);
  if (!ptr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess) return nullptr;
    ptr[dev] = static_cast<float*>(p);
  }
  return ptr[dev];
}

int lmk_xent_noalloc(int precision, void* z, int64_t ldz, int M, int V, const int32_t* tgt, float* loss,
                     uint32_t* flags, const float* loss_scale, void* stream) {
  if (M <= 0 || M > kXentNoallocRows || V <= 0 || ldz < V || ldz % 8 || precision < 0 || precision > 2) return -1;
  if (!z || !tgt || !loss || !flags) return -1;
  float* sp = xent_scratch();
  if (!sp) return -2;
  // the count and every row's loss are written before they are read: nothing
  // to clear
  return lmk_xent(precision, z, ldz, M, V, tgt, loss, reinterpret_cast<int32_t*>(sp), sp + kXentNoallocHead, flags,
                  loss_scale, stream);
}

int lmk_csr(const int32_t* keys, int M, int nkeys, int32_t* counts, int32_t* offsets, int32_t* chunk_base,
            int32_t* perm, int32_t* rank, void* stream) {
  if (M < 0 || nkeys <= 0 || (M > 0 && !rank)) return -1;
  auto a16 = [](const void* q) { return reinterpret_cast<uintptr_t>(q) % 16 == 0; };
  if (!a16(counts) || !a16(offsets) || !a16(chunk_base)) return -1;
  EmbedBwdWs w{counts, offsets, chunk_base, perm, nullptr, rank, csr_rank_ints(M, nkeys)};
  launch_csr(keys, M, nkeys, w, S(stream));
  return 0;
}

int64_t lmk_csr_ws_ints(int M, int nkeys) { return M < 0 || nkeys <= 0 ? -1 : csr_rank_ints(M, nkeys); }

int64_t lmk_segment_sum_ws_floats(int M, int nkeys, int C) { return embed_bwd_max_chunks(M, nkeys) * C; }

int lmk_segment_sum(const float* dx, int M, int C, int nkeys, int32_t* counts, int32_t* offsets, int32_t* chunk_base,
                    int32_t* perm, float* partial, float* dst, int accumulate, void* stream) {
  if (M < 0 || nkeys <= 0 || C <= 0) return -1;
  EmbedBwdWs w{counts, offsets, chunk_base, perm, partial, nullptr};
  launch_segment_sum(dx, nullptr, M, C, nkeys, w, dst, accumulate != 0, S(stream));
  return 0;
}

int lmk_grad_norm(const float* g, int64_t n, float clip, double* part, float* norm_scale, uint32_t* flags,
                  float* scale_state, float growth, float backoff, int interval, void* stream) {
  if (n < 0 || (scale_state && (interval < 1 || !(growth >= 1.f) || !(backoff > 0.f)))) return -1;
  LossScaler ls;
  ls.state = scale_state;
  ls.growth = growth;
  ls.backoff = backoff;
  ls.interval = interval;
  launch_sumsq_partials(g, n, part, S(stream));
  launch_norm_finalize(part, clip, norm_scale, flags, nullptr, ls, S(stream));
  return 0;
}

int lmk_adamw(float* p, const float* g, float* m, float* v, int64_t n, float lr, float beta1, float beta2, float eps,
              float weight_decay, int step, const float* norm_scale, const uint32_t* flags, uint16_t* shadow,
              int shadow_f16, void* stream) {
  if (n < 0 || n % 4 || step < 1) return -1;
  AdamArgs a{};
  a.p = p; a.g = g; a.m = m; a.v = v; a.n = n;
  a.lr = lr; a.beta1 = beta1; a.beta2 = beta2; a.eps = eps; a.wd = weight_decay;
  a.bc1 = (float)(1.0 - std::pow((double)beta1, (double)step));
  a.bc2 = (float)(1.0 - std::pow((double)beta2, (double)step));
  a.norm_scale = norm_scale; a.flags = flags; a.shadow = shadow; a.shadow_f16 = shadow_f16 != 0;
  launch_adamw(a, S(stream));
  return 0;
}

}  // extern "C"

#undef ACT_T
