// Internal launch interface of the gfx950 kernels (host side).
#pragma once

#include "common.h"

namespace lm {

constexpr int kLnRowsPerBlock = 16;  // rows per block in the LayerNorm backward
constexpr int kColRows = 128;        // rows per partial in the bias-gradient column sums

// ------------------------------------------------------------------- GEMM
// C[i, j] = sum_k A(i, k) B(j, k) for i < M, j < N, k < K, then an epilogue.
// A(i, k) = A[i * lda + k] when a_kc (K-contiguous) else A[k * lda + i];
// B(j, k) = B[j * ldb + k] when b_kc else B[k * ldb + j].
//   forward  Y = X W^T : a_kc, b_kc
//   dX = dY W          : a_kc, !b_kc
//   dW = dY^T X        : !a_kc, !b_kc
enum GemmEpi : int {
  EPI_STORE = 0,    // C = acc (+ bias[j]); C fp32 or activation type
  EPI_RESID = 1,    // C fp32 = R[i, j] + acc (+ bias[j])
  EPI_GELU = 2,     // u = acc + bias[j]: C (act) = GELU'(u), aux (act) = GELU(u)
  EPI_DGELU = 3,    // C (act) = acc * aux[i, j] (aux: the GELU' the forward stored)
  EPI_PARTIAL = 4,  // C fp32 [split][M][ldc] = acc (split-K partial sums)
};

struct GemmOp {
  int M = 0, N = 0, K = 0;
  const void* A = nullptr;
  long lda = 0;
  bool a_kc = true;
  const void* B = nullptr;
  long ldb = 0;
  bool b_kc = true;
  void* C = nullptr;
  long ldc = 0;
  int epi = EPI_STORE;
  bool c_f32 = false;  // EPI_STORE output type
  const float* bias = nullptr;
  const float* R = nullptr;
  long ldr = 0;
  void* aux = nullptr;
  long ld_aux = 0;
  int force_split = 0;  // > 0: use exactly this many K splits (tests)
  int M_out = 0;        // > 0: store only rows < M_out (rows M_out..M-1 are padding)
  // EPI_DGELU, 16-bit, where gemm16_colsum_rows says the kernel writes them:
  // the column sums of the output (fp32, before rounding) over each 64-row
  // half of each 128-row block; row 2b + h of colsum [2 ceil(M / 128)][N]
  // holds rows 128 b + 64 h .. + 63.
  float* colsum = nullptr;
  // > 0: this tile configuration instead of the dispatcher's choice (16-bit
  // path; tests and measurements); an unknown one, or one that does not run
  // the op's layout and epilogue, is rejected
  int cfg = 0;
};

// Returns 0 or a negative code if the shape breaks the kernel's alignment
// rules (leading dims and K-contiguous K multiples of 8, M/N multiples of 8
// for the non-K-contiguous operands).
int gemm_bf16(const GemmOp& op, float* ws, long ws_floats, hipStream_t s);
int gemm_f16(const GemmOp& op, float* ws, long ws_floats, hipStream_t s);
int gemm_f32(const GemmOp& op, float* ws, long ws_floats, hipStream_t s);
// 0 if the dispatcher of the 16-bit (h16) or fp32 path accepts op, else -1:
// the checks the launch itself makes, without launching (no pointer is read).
int gemm_check(const GemmOp& op, bool h16);
// Split-K partial floats the op's launch configuration would use (0: no split);
// with a smaller workspace the GEMM runs unsplit.
long gemm_ws_floats_needed(const GemmOp& op, bool h16);
// Split count the 16-bit dispatcher would pick (for workspace sizing).
int gemm16_splits(const GemmOp& op);
// Rows of GemmOp::colsum the 16-bit dispatcher's kernel writes for op, or 0
// where it cannot (then colsum must stay null).
int gemm16_colsum_rows(const GemmOp& op);

// Grouped launch of weight-gradient GEMMs (16-bit operands, both M/N-major,
// fp32 output, plain store, no bias): gemm_group_plan fills a table of
// gemm_group_table_bytes(n) bytes in host memory for ops[0..n) and returns
// the launch's unit count (-1: an op the grouped kernel does not take), with
// the tile width in *tn; gemm_group_launch runs the launch from a device copy
// of that table. Each output element is one unit's fixed-order sum over K.
long gemm_group_table_bytes(int n);
// part (nullable): per op, the fp32 partial-sum buffer of an op with
// force_split = s > 1, which then runs in K slices of whole 64-value steps
// ([slices][M][N]; gemm_group_slices_of gives the count) to be summed by
// launch_group_reduce; other ops store their result directly.
int gemm_group_plan(const GemmOp* ops, int n, void* table, int* tn, float* const* part = nullptr);
int gemm_group_slices_of(const GemmOp& op);
constexpr int kGroupReduceMax = 32;
struct GroupReduce {
  int n;
  const float* part[kGroupReduceMax];
  float* dst[kGroupReduceMax];
  int rows[kGroupReduceMax], cols[kGroupReduceMax], S[kGroupReduceMax];
  long ldc[kGroupReduceMax], stride[kGroupReduceMax];
};
void launch_group_reduce(const GroupReduce& gr, hipStream_t s);
int gemm_group_launch(bool f16_ops, int tn, const void* table_dev, int units, hipStream_t s);
// compute units of the current device
int gemm_cus();

// -------------------------------------------------------------- rows etc.
void launch_fill_u32(uint32_t* p, uint32_t v, long n, hipStream_t s);
void launch_index_layout(const int32_t* doc, int B, int T, int32_t* start, int32_t* end, int32_t* pos,
                         uint32_t* flags, hipStream_t s);
void launch_embed_fwd(const int32_t* tok, const int32_t* pos, const float* wte, const float* wpe, int M, int C,
                      int V, float* x, uint32_t* flags, hipStream_t s);
void launch_count_valid(const int32_t* tgt, int M, int V, int32_t* n_out, float* stats, uint32_t* flags,
                        hipStream_t s);
void launch_loss_reduce(const float* row_loss, int M, const int32_t* n_valid, float* out, hipStream_t s);
void launch_write_flags(const uint32_t* flags, float* stats, hipStream_t s);
template <typename T>
void launch_f32_to(const float* src, T* dst, long n, hipStream_t s);
template <typename T>
void launch_logits_out(const T* z, long ldz, int M, int V, float* out, hipStream_t s);

template <typename T>
void launch_ln_fwd(const float* x, const float* g, const float* b, int M, int C, float eps, T* y, float* mu,
                   float* rstd, hipStream_t s);
template <typename T>
void launch_ln_bwd(const float* dy, const float* x, const float* mu, const float* rstd, const float* g, int M,
                   int C, const float* g_in, float* g_out, T* g_act, float* part_dg, float* part_db,
                   float* part_dc, hipStream_t s);
void launch_colsum_partials(const float* pa, const float* pb, int P, int C, float* oa, float* ob, hipStream_t s,
                            const float* pc = nullptr, float* oc = nullptr);
// Up to kColsumBatch reductions of the same shape (P partial rows, C
// columns) in one launch; set i reads pa/pb/pc[i] and writes oa/ob/oc[i]
// (pb, pc, ob, oc may be null).
constexpr int kColsumBatch = 32;
struct ColsumBatch {
  const float* pa[kColsumBatch];
  const float* pb[kColsumBatch];
  const float* pc[kColsumBatch];
  float* oa[kColsumBatch];
  float* ob[kColsumBatch];
  float* oc[kColsumBatch];
};
void launch_colsum_partials_batch(const ColsumBatch& bt, int n, int P, int C, hipStream_t s);
// Per-row-block partial column sums (as launch_colsum_stage1) of n <=
// kColsumBatch 16-bit matrices of one shape [M, N] (leading dimension lda;
// N and lda multiples of 8) in one launch, matrix i into part[i].
struct Colsum16Batch {
  const void* a[kColsumBatch];
  float* part[kColsumBatch];
};
template <typename T>
void launch_colsum_stage1_batch(const Colsum16Batch& b, int n, long lda, int M, int N, hipStream_t s);
template <typename T>
void launch_colsum(const T* a, long lda, int M, int N, float* part, float* out, hipStream_t s);
// Its first stage alone: the (M / kColRows rounded up) x N partial rows,
// reduced later (launch_colsum_partials[_batch]).
template <typename T>
void launch_colsum_stage1(const T* a, long lda, int M, int N, float* part, hipStream_t s);

// loss_scale (nullable, device): dz is multiplied by *loss_scale.
template <typename T>
void launch_xent(T* z, long ldz, int M, int V, const int32_t* tgt, const int32_t* n_valid, float* row_loss,
                 const float* loss_scale, hipStream_t s);

// -------------------------------------------------------------- attention
// qkv [B*T, 3C] (q | k | v, head h in columns h*D..h*D+D-1 of each third),
// o [B*T, C], lse [B, H, T] (natural log), start/end [B, T].
struct AttnArgs {
  const void* qkv;
  const int32_t* start;
  const int32_t* end;
  int B, T, H, D;
  void* o;
  float* lse;
  // backward
  const void* dout;  // [B*T, C]
  float* delta;      // [B, H, T] rowsum(dO * O)
  void* dqkv;        // [B*T, 3C]
};
// E: bf16 or f16 operands (matrix cores); the fp32 path has its own kernels.
template <typename E>
int attn_fwd16(const AttnArgs& a, hipStream_t s);
int attn_fwd_f32(const AttnArgs& a, hipStream_t s);
// Backward in three launches: delta = rowsum(dO * O), the dQ pass, the dK/dV
// pass (part 0, 1, 2); attn_bwd* runs all three. The 16-bit dQ pass computes
// delta itself (part 0 launches nothing there).
template <typename E>
int attn_bwd_part16(const AttnArgs& a, int part, hipStream_t s);
int attn_bwd_part_f32(const AttnArgs& a, int part, hipStream_t s);
template <typename E>
int attn_bwd16(const AttnArgs& a, hipStream_t s);
int attn_bwd_f32(const AttnArgs& a, hipStream_t s);

// ------------------------------------------------------ embedding backward
// Deterministic scatter-add: a stable counting sort of the keys (token ids,
// then positions) gives each key's rows in ascending index order; rows are
// summed in that order, in chunks of kSegRows, and the chunks of one key are
// added in order.
constexpr int kSegRows = 64;
struct EmbedBwdWs {
  int32_t* counts;     // [nkeys + 1]
  int32_t* offsets;    // [nkeys + 1]
  int32_t* chunk_base; // [nkeys + 1]
  int32_t* perm;       // [M]
  float* partial;      // [max_chunks, C]
  int32_t* rank;       // scratch of the sort: at least M ints, rank_cap in all
  long rank_cap = 0;   // ints at rank (0: M)
};
// Ints of sort scratch with which launch_csr takes its linear-time rank for
// up to M rows (M when it keeps the pairwise one).
long csr_rank_ints(int M, int nkeys);
void launch_csr(const int32_t* keys, int M, int nkeys, EmbedBwdWs ws, hipStream_t s);
// dst[key] (+)= sum of dx rows of that key. accumulate: add onto dst (rows of
// keys with no occurrence are left untouched) else overwrite (zero rows for
// absent keys).
void launch_segment_sum(const float* dx, const int32_t* keys, int M, int C, int nkeys, EmbedBwdWs ws, float* dst,
                        bool accumulate, hipStream_t s);
long embed_bwd_max_chunks(int M, int nkeys);
// dst[t] = sum over b of dx rows b T + t (t < T), zero for T <= t < S: the
// position gradient of rows without packed documents, summed in the order of
// launch_segment_sum (bit-identical to it); C a multiple of 4.
void launch_pos_colsum(const float* dx, int B, int T, int C, int S, float* dst, hipStream_t s);

// --------------------------------------------------------------- optimiser
constexpr int kNormBlocks = 1024;
void launch_sumsq_partials(const float* g, long n, double* part, hipStream_t s);
// Dynamic loss scale of fp16 training: state[0] = S, state[1] = finite steps
// in a row (device memory, updated by launch_norm_finalize); state = nullptr
// means no scaling.
struct LossScaler {
  float* state = nullptr;
  float growth = 2.f, backoff = 0.5f;
  int interval = 2000;
};
// Final norm: the partial sums are of (S g)^2; n = sqrt(sum) / S, stats[1] =
// n; clip factor c = clip/n if n > clip > 0 else 1; norm_scale = [n, c / S];
// sets flags bit 0 if n is not finite; then updates the loss scale.
void launch_norm_finalize(const double* part, float clip, float* norm_scale, uint32_t* flags, float* stats,
                          LossScaler ls, hipStream_t s);
struct AdamArgs {
  float* p;
  const float* g;
  float* m;
  float* v;
  long n;
  float lr, beta1, beta2, eps, wd;
  float bc1, bc2;  // 1 - beta1^t, 1 - beta2^t
  const float* norm_scale;  // [norm, scale]
  const uint32_t* flags;
  uint16_t* shadow;  // 16-bit copy of p at the same offsets (nullable)
  int shadow_f16;    // the copy is fp16 (else bf16)
};
void launch_adamw(const AdamArgs& a, hipStream_t s);
void launch_make_shadow(const float* p, long n, uint16_t* shadow, bool to_f16, hipStream_t s);

// ------------------------------------------------------------- generation
// Key/value cache (per layer K [B][S][C] then V [B][S][C]): rows t0 .. t0+T-1
// of each row b from qkv [B*T, 3C]; one query per (row, head) against cache
// positions 0 .. n-1 (sbuf: B*H*S floats of scratch).
// d_pos (nullable): the generation position in device memory, read when the
// kernels run (so a captured graph can be replayed at later positions),
// clamped to [1, S-1]; it then replaces t0 (kv_store) and n = pos + 1.
template <typename E>
void launch_kv_store(const E* qkv, int B, int T_, int C, int S, int t0, E* kc, E* vc, hipStream_t s,
                     const int32_t* d_pos = nullptr);
template <typename T>
int launch_attn_decode(const T* qkv, const T* kc, const T* vc, int B, int H, int D, int S, int n, T* o, float* sbuf,
                       hipStream_t s, const int32_t* d_pos = nullptr);
// dst[0 .. n-1] = *d_pos clamped to [1, S-1]
void launch_fill_pos(int32_t* dst, const int32_t* d_pos, int S, long n, hipStream_t s);
__device__ __forceinline__ int decode_pos(const int32_t* d_pos, int S) {
  const int p = *d_pos;
  return p < 1 ? 1 : (p > S - 1 ? S - 1 : p);
}
// Next token of each of `rows` logit rows (row r at logits + r * ld, V
// columns): greedy when temperature <= 0, else top-k sampling with the given
// uniforms; out [rows].
void launch_sample(const float* logits, int rows, int V, long ld, float temperature, int top_k, const float* u,
                   int32_t* out, hipStream_t s);

}  // namespace lm
