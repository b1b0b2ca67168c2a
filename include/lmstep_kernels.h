/*
 * lmstep_kernels.h - per-kernel C ABI of the training-step library.
 *
 * These entry points launch one kernel (or one short fixed sequence) of the
 * step on caller-provided device buffers, so each can be checked on its own
 * against the CPU oracle. They are the same kernels train_step launches.
 * All pointers are device pointers unless stated; stream is a hipStream_t as
 * void*; every call only enqueues work and returns 0, or a negative value if
 * the shape breaks the kernel's rules (nothing is enqueued then).
 * precision: 0 = fp32 activations (float), 1 = bf16 activations (uint16_t
 * storage of bfloat16), 2 = fp16 activations (IEEE binary16). Statistics,
 * residuals and gradients stay fp32.
 */
#ifndef LMSTEP_KERNELS_H
#define LMSTEP_KERNELS_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Epilogues of lmk_gemm. */
enum { LMK_EPI_STORE = 0, LMK_EPI_RESID = 1, LMK_EPI_GELU = 2, LMK_EPI_DGELU = 3 };

/* C[i,j] = sum_k A(i,k) B(j,k), i < M, j < N, k < K (the dense products of
 * the step: Y = X W^T, dX = dY W, dW = dY^T X), then the epilogue:
 *   STORE: C = acc + bias[j]              (C fp32 if c_f32, else activation type)
 *   RESID: C (fp32) = R[i,j] + acc + bias[j]  (residual add of a block)
 *   GELU : u = acc + bias[j]; C = GELU'(u), aux = GELU(u), tanh form (Feste
 *          page, "Model Architecture": GELU activation); the derivative is
 *          stored for the backward's DGELU
 *   DGELU: C = acc * aux[i,j]  (aux: the GELU'(u) a GELU epilogue stored)
 * A(i,k) = A[i*lda + k] if a_kc else A[k*lda + i]; B(j,k) = B[j*ldb + k] if
 * b_kc else B[k*ldb + j]. bias may be NULL. Rows >= M_out (if 0 < M_out < M)
 * are computed but not stored. force_split > 0 forces that many K slices
 * (summed in slice order); ws is an fp32 scratch of ws_floats for them.
 * bf16 rules: lda, ldb multiples of 8; K a multiple of 8 when an operand is
 * K-contiguous; M (N) a multiple of 8 when A (B) is not; N and the output
 * leading dimensions multiples of 8; each operand spans less than 2 GiB
 * (its loads use 32-bit byte offsets); an output tile of 256 rows spans less
 * than 2 GiB. */
int lmk_gemm(int precision, int M, int N, int K, const void* A, int64_t lda, int a_kc, const void* B, int64_t ldb,
             int b_kc, void* C, int64_t ldc, int epi, int c_f32, const float* bias, const float* R, int64_t ldr,
             void* aux, int64_t ld_aux, int force_split, int M_out, float* ws, int64_t ws_floats, void* stream);

/* lmk_gemm with an explicit tile configuration of the 16-bit path instead of
 * the dispatcher's choice (cfg 0 = the dispatcher's choice), for tests that
 * must run a given kernel and for measurements: 1 = 128 x 128 register-staged
 * kernel, 11 = persistent 256 x 256, 12 = persistent 128 x 128, 14 =
 * persistent 192 x 128 (K-contiguous operands and a 16-bit plain store only),
 * 15 / 16 = persistent K-split kernel at 128 x 192 / 128 x 128 (eight
 * wavefronts, one block per CU).
 * Rejected (-1, nothing enqueued): an unknown cfg, one that does not run the
 * layout and epilogue asked for, any cfg > 0 with precision 0. */
int lmk_gemm_cfg(int cfg, int precision, int M, int N, int K, const void* A, int64_t lda, int a_kc, const void* B,
                 int64_t ldb, int b_kc, void* C, int64_t ldc, int epi, int c_f32, const float* bias, const float* R,
                 int64_t ldr, void* aux, int64_t ld_aux, int force_split, int M_out, float* ws, int64_t ws_floats,
                 void* stream);

/* The weight gradients of several linear layers in one launch (Feste page,
 * "Manual Backpropagation": dW = dY^T X per layer), as the training step runs
 * those of its blocks: problem i (i < n) computes C_i[r,c] = sum_k
 * A_i[k*lda_i + r] B_i[k*ldb_i + c], r < M_i, c < N_i, k < K_i, with
 * (M_i, N_i, K_i) = mnk[3i], mnk[3i+1], mnk[3i+2]; A_i and B_i 16-bit
 * (precision 1 bf16, 2 fp16), C_i fp32 (overwritten, leading dimension ldc_i).
 * Each output element is one fixed-order sum over k (bit-identical between
 * runs). table: a device buffer of at least lmk_gemm_group_table_bytes(n)
 * bytes that the call fills (the stream is synchronized first); it must not
 * be reused until the launch has run. Rules per problem as lmk_gemm's for a
 * dW layout (both operands not K-contiguous). Returns -1 with nothing
 * enqueued on a bad argument or a problem the grouped kernel does not take. */
int64_t lmk_gemm_group_table_bytes(int n);
int lmk_gemm_group(int precision, int n, const int* mnk, const void* const* A, const int64_t* lda,
                   const void* const* B, const int64_t* ldb, float* const* C, const int64_t* ldc, void* table,
                   int64_t table_bytes, void* stream);

/* LayerNorm over rows of x [M,C] fp32 (biased variance): y = g (x-mu) rstd + b
 * (y in the activation type), mu and rstd [M] fp32 (RustGPT page, file list:
 * layer_norm). C a multiple of 128, at most 1024. */
int lmk_layernorm_fwd(int precision, const float* x, const float* g, const float* b, int M, int C, float eps, void* y,
                      float* mu, float* rstd, void* stream);

/* LayerNorm backward: g_out = g_in + dx (g_in may be NULL or equal g_out),
 * g_act (nullable) = g_out in the activation type, dgamma/dbeta [C] fp32
 * (overwritten), dsum (nullable) [C] fp32 = column sums of g_out (the
 * gradient of a bias added to the LayerNorm's input). ws: fp32 scratch of
 * lmk_layernorm_bwd_ws_floats(M, C). */
int lmk_layernorm_bwd(int precision, const float* dy, const float* x, const float* mu, const float* rstd,
                      const float* g, int M, int C, const float* g_in, float* g_out, void* g_act, float* dgamma,
                      float* dbeta, float* dsum, float* ws, void* stream);
int64_t lmk_layernorm_bwd_ws_floats(int M, int C);

/* Column sums of an [M,N] matrix (bias gradients) into out [N] fp32, summed
 * in a fixed order. ws: fp32 scratch of lmk_colsum_ws_floats(M, N). */
int lmk_colsum(int precision_of_a, const void* a, int64_t lda, int M, int N, float* out, float* ws, void* stream);
int64_t lmk_colsum_ws_floats(int M, int N);

/* Packed-row index layout (LucilleAI page, sequence packing): for doc ids
 * [B,T] (NULL: one document per row) writes start, end, pos [B,T] int32;
 * flags bit 1 is set if doc ids decrease along a row. */
int lmk_index_layout(const int32_t* doc, int B, int T, int32_t* start, int32_t* end, int32_t* pos, uint32_t* flags,
                     void* stream);

/* x[m,:] = wte[tok[m],:] + wpe[pos[m],:] (Feste page, "Model Architecture"). */
int lmk_embed_fwd(const int32_t* tok, const int32_t* pos, const float* wte, const float* wpe, int M, int C, int V,
                  float* x, uint32_t* flags, void* stream);

/* Causal (block-diagonal with start/end) multi-head attention over
 * qkv [B*T, 3C] -> o [B*T, C], lse [B,H,T] natural-log row log-sum-exp
 * (Feste page, "Model Architecture": -inf mask before the softmax). */
int lmk_attn_fwd(int precision, const void* qkv, const int32_t* start, const int32_t* end, int B, int T, int H, int D,
                 void* o, float* lse, void* stream);
/* Backward: dqkv [B*T, 3C] from dout [B*T, C]; delta [B,H,T] fp32 scratch. */
int lmk_attn_bwd(int precision, const void* qkv, const void* o, const float* lse, const void* dout,
                 const int32_t* start, const int32_t* end, int B, int T, int H, int D, float* delta, void* dqkv,
                 void* stream);

/* Softmax cross-entropy over z [M, ldz] (V valid columns, ldz a multiple of
 * 8) and targets [M] (-1 = ignored): loss[0] = mean over valid rows of
 * lse - z[tgt]; z is overwritten with dz = (softmax - onehot)/N (0 on ignored
 * rows and padding columns); loss[3] = N. ws: int32 [4] + fp32 [M] scratch.
 * loss_scale (nullable, one device float S): dz is multiplied by S (the
 * gradient of S times the loss, for fp16 training with loss scaling, the
 * LucilleAI page's GradScaler); the loss is not. */
int lmk_xent(int precision, void* z, int64_t ldz, int M, int V, const int32_t* tgt, float* loss, int32_t* ws_n,
             float* ws_rows, uint32_t* flags, const float* loss_scale, void* stream);

/* lmk_xent for callers that cannot allocate (code under HIP graph capture,
 * tight serving loops, harnesses that forbid allocation): the same kernels,
 * with the valid-target count and the per-row losses in a static device
 * buffer of this library instead of ws_n / ws_rows. The buffer holds
 * 65536 rows (M > 65536: -1, nothing enqueued) and about 256 KB per GPU the
 * library runs on, kept until the process ends; its address is looked up
 * once per GPU on the first call there. The call allocates nothing. Calls
 * that overlap on one GPU (on different streams) share the buffer and race;
 * the count and every row's loss are rewritten by each call, so nothing
 * carries over from one call to the next. -2 if the buffer's address cannot
 * be obtained. */
int lmk_xent_noalloc(int precision, void* z, int64_t ldz, int M, int V, const int32_t* tgt, float* loss,
                     uint32_t* flags, const float* loss_scale, void* stream);

/* Stable counting sort of keys [M] in [0, nkeys): counts/offsets/chunk_base
 * [nkeys+1], 16-byte aligned, perm [M] (rows of key v at
 * perm[offsets[v] .. offsets[v+1]), ascending); rank: int32 scratch of
 * lmk_csr_ws_ints(M, nkeys) entries (each row's count of equal keys before
 * it: M entries when it is counted pairwise, a [blocks of 256 rows][nkeys]
 * table of per-block counts from 128 blocks on). -1 on a bad size or
 * alignment. */
int lmk_csr(const int32_t* keys, int M, int nkeys, int32_t* counts, int32_t* offsets, int32_t* chunk_base,
            int32_t* perm, int32_t* rank, void* stream);
int64_t lmk_csr_ws_ints(int M, int nkeys);
/* dst[v,:] (+)= sum of dx rows with key v, in perm order (after lmk_csr).
 * partial: fp32 scratch of lmk_segment_sum_ws_floats(M, nkeys, C). */
int lmk_segment_sum(const float* dx, int M, int C, int nkeys, int32_t* counts, int32_t* offsets,
                    int32_t* chunk_base, int32_t* perm, float* partial, float* dst, int accumulate, void* stream);
int64_t lmk_segment_sum_ws_floats(int M, int nkeys, int C);

/* Global L2 norm of g [n] and the clip factor: norm_scale = [n, s], s =
 * clip/n if n > clip > 0 else 1 (RustGPT page: clip to L2 norm 5.0); flags
 * bit 0 if n is not finite. part: double scratch [1024].
 * scale_state (nullable, device float[2] = [S, finite steps in a row]): g
 * holds S times the gradient; then n is the norm of g divided by S,
 * norm_scale[1] = s / S, and the state follows the dynamic loss-scale rule
 * (LucilleAI page: GradScaler): a non-finite n sets S = S * backoff and the
 * count to 0; otherwise the count grows by one, and on reaching `interval`
 * S = S * growth and the count is 0. Without a state, growth, backoff and
 * interval are ignored. */
int lmk_grad_norm(const float* g, int64_t n, float clip, double* part, float* norm_scale, uint32_t* flags,
                  float* scale_state, float growth, float backoff, int interval, void* stream);

/* AdamW with decoupled weight decay (Feste page, "Manual Backpropagation")
 * on n elements (n a multiple of 4), gradient scaled by norm_scale[1];
 * skipped entirely when flags bit 0 is set; shadow (nullable) gets p rounded to
 * fp16 (shadow_f16 = 1) or bf16 (0). */
int lmk_adamw(float* p, const float* g, float* m, float* v, int64_t n, float lr, float beta1, float beta2, float eps,
              float weight_decay, int step, const float* norm_scale, const uint32_t* flags, uint16_t* shadow,
              int shadow_f16, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* LMSTEP_KERNELS_H */
