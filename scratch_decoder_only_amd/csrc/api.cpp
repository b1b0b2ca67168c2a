// Host side of the C ABI: configuration checks, the parameter table, carving
// of the caller's arena, and the fixed kernel sequence of one training step.
// Everything is enqueued on the caller's stream; the library never allocates
// device memory.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <string>
#include <type_traits>
#include <vector>

#include "../../include/lmstep.h"
#include "host.h"
#include "kernels.h"

using namespace lm;

namespace {

thread_local std::string g_err;

lm_status fail(lm_status st, const std::string& msg) {
  g_err = msg;
  return st;
}

}  // namespace

// Error message for the other host files of the library (checkpoint I/O).
lm_status lm::set_error(lm_status st, const std::string& msg) { return fail(st, msg); }

namespace {

constexpr size_t kAlign = 256;

size_t align_up(size_t v, size_t a) { return (v + a - 1) / a * a; }
long round_up(long v, long a) { return (v + a - 1) / a * a; }

struct Carver {
  char* base;
  size_t off = 0;
  template <typename T>
  T* take(size_t n) {
    off = align_up(off, kAlign);
    T* p = base ? reinterpret_cast<T*>(base + off) : nullptr;
    off += n * sizeof(T);
    return p;
  }
};

struct TensorInfo {
  std::string name;
  long off, rows, cols;
};

// Per-class event timing of kernel launches (measurement hook).
struct Profiler {
  bool on = false;
  struct Cls {
    std::string name;
    long launches = 0;
    double ms = 0, flops = 0, bytes = 0;
  };
  std::vector<Cls> cls;
  struct Pending {
    int cls;
    hipEvent_t a, b;
  };
  std::vector<Pending> pending;
  std::vector<hipEvent_t> pool;
  size_t pool_used = 0;

  int find(const char* name) {
    for (size_t i = 0; i < cls.size(); ++i)
      if (cls[i].name == name) return (int)i;
    cls.push_back(Cls{name});
    return (int)cls.size() - 1;
  }
  hipEvent_t take() {
    if (pool_used == pool.size()) {
      hipEvent_t e;
      if (hipEventCreate(&e) != hipSuccess) return nullptr;
      pool.push_back(e);
    }
    return pool[pool_used++];
  }
  void drain() {
    if (pending.empty()) return;
    (void)hipEventSynchronize(pending.back().b);
    for (auto& p : pending) {
      float ms = 0;
      if (hipEventElapsedTime(&ms, p.a, p.b) == hipSuccess) cls[p.cls].ms += ms;
    }
    pending.clear();
    pool_used = 0;
  }
  ~Profiler() {
    for (auto e : pool) (void)hipEventDestroy(e);
  }
};

}  // namespace

struct lm_model {
  lm_config cfg;
  int V, C, H, D, F, L, S, Bmax;
  int prec;  // 0 fp32, 1 bf16, 2 fp16 (with dynamic loss scaling)
  bool h16;  // 16-bit operands (bf16 or fp16)
  bool untied;  // separate vocabulary projection head.w [V, C] with bias head.b [V]
  long Vp;   // padded vocabulary (columns of the logits; rows reserved for wte and head.w)
  long ldz;  // leading dimension of the logits
  std::vector<TensorInfo> table;
  long P = 0;  // floats in the flat parameter buffer
  // tensor offsets
  long o_wte, o_wpe, o_lnf_g, o_lnf_b, o_head_w, o_head_b;
  struct Blk {
    long ln1_g, ln1_b, w_qkv, b_qkv, w_o, b_o, ln2_g, ln2_b, w_fc, b_fc, w_proj, b_proj;
  };
  std::vector<Blk> blk;
  size_t act_size;  // bytes of one activation element
  // arena slices
  float *params, *grads, *adam_m, *adam_v;
  uint16_t* shadow;  // 16-bit copy of the flat parameter buffer (bf16 or fp16 path)
  float* x;      // [L+1][M][C]
  float* xm;     // [L][M][C]
  // gelu_d: GELU'(u) of each block's MLP-in pre-activation u, which the
  // forward's GELU epilogue stores beside GELU(u) for the backward
  char *y1, *qkv, *o, *y2, *gelu_d, *a, *hf, *logits;
  float *mu1, *r1, *mu2, *r2, *muf, *rf, *lse;
  float *g, *dy, *delta;
  char *g_act, *dbig, *dO;
  // The per-layer weight gradients of the 16-bit path, when the model has
  // enough of their tiles to fill the CUs several times over, run as one
  // grouped launch after the backward (no K slices, no reduction passes, one
  // launch's fixed cost): the output gradients they read are kept per layer
  // (g_act_l: the two LayerNorm-backward outputs of each block, du_l: the
  // MLP-in pre-activation gradient, dqkv_l: the QKV gradient), and dw_tab is
  // the launch's table on the device, dw_tab_host its last uploaded image.
  bool dw_group = false;
  // K slices of every GEMM of the grouped launch (1: whole K per unit) and
  // their partial sums
  int dw_slices = 1;
  float* dw_part = nullptr;
  char *g_act_l = nullptr, *du_l = nullptr, *dqkv_l = nullptr, *dw_tab = nullptr;
  std::vector<char> dw_tab_host;
  float *ln_part, *col_part, *bias_part, *gemm_ws;
  long gemm_ws_floats;
  EmbedBwdWs emb_tok, emb_pos;
  int32_t *start, *end, *pos, *n_valid;
  uint32_t* flags;
  float *row_loss, *norm_scale, *stats_own;
  float* scale_state;                 // fp16: [loss scale S, finite steps in a row]
  float ls_growth = 2.f, ls_backoff = 0.5f;
  int ls_interval = 2000;
  double* norm_part;
  size_t bytes = 0;
  Profiler prof;

  long M() const { return (long)Bmax * S; }
  const float* P_(long off) const { return params + off; }
  template <typename T>
  T* act(char* base, long elem_off) const {
    return reinterpret_cast<T*>(base + elem_off * act_size);
  }
  // operand copy of a weight: the 16-bit copy (bf16 or fp16 path) or the fp32 master
  const void* W(long off) const { return h16 ? static_cast<const void*>(shadow + off) : params + off; }
  // the vocabulary projection's weight (wte when tied)
  long head_w() const { return untied ? o_head_w : o_wte; }
  // the dynamic loss scale (fp16 only)
  LossScaler scaler() const {
    LossScaler ls;
    if (prec == 2) {
      ls.state = scale_state;
      ls.growth = ls_growth;
      ls.backoff = ls_backoff;
      ls.interval = ls_interval;
    }
    return ls;
  }
};

namespace {

lm_status validate(const lm_config* c) {
  if (!c) return fail(LM_ERR_ARG, "config is NULL");
  if (c->vocab < 1 || c->d_model < 1 || c->n_heads < 1 || c->d_mlp < 1 || c->n_layers < 0 || c->max_seq < 1 ||
      c->max_batch < 1)
    return fail(LM_ERR_SHAPE, "model dimensions must be positive (n_layers >= 0)");
  if (c->d_model % c->n_heads) return fail(LM_ERR_SHAPE, "d_model must be a multiple of n_heads");
  if (c->d_model % 128 || c->d_model > 1024)
    return fail(LM_ERR_UNSUPPORTED, "d_model must be a multiple of 128 and at most 1024");
  int D = c->d_model / c->n_heads;
  if (D != 32 && D != 64) return fail(LM_ERR_UNSUPPORTED, "head dimension must be 32 or 64");
  if (c->d_mlp % 64) return fail(LM_ERR_UNSUPPORTED, "d_mlp must be a multiple of 64");
  if (c->precision < 0 || c->precision > 2)
    return fail(LM_ERR_ARG, "precision must be 0 (fp32), 1 (bf16) or 2 (fp16 with loss scaling)");
  if (c->untied_head != 0 && c->untied_head != 1) return fail(LM_ERR_ARG, "untied_head must be 0 or 1");
  if (!(c->ln_eps >= 0.f)) return fail(LM_ERR_ARG, "ln_eps must be >= 0");
  if ((long)c->max_batch * c->max_seq > (1L << 24)) return fail(LM_ERR_SHAPE, "max_batch * max_seq too large");
  return LM_OK;
}

// The vocabulary-sized tensors reserve Vp rows (and the head bias ldz
// entries): the padding stays zero, so the GEMMs and the bf16 copy can treat
// them as Vp x C without a separate padded buffer.
void build_table(lm_model* m) {
  auto add = [&](const std::string& n, long rows, long cols, long reserve = 0) {
    long off = m->P;
    m->table.push_back({n, off, rows, cols});
    m->P = round_up(off + std::max(rows * cols, reserve), 64);
    return off;
  };
  const int V = m->V, C = m->C, F = m->F, S = m->S;
  m->o_wte = add("wte", V, C, m->Vp * C);
  m->o_wpe = add("wpe", S, C);
  m->blk.resize(m->L);
  for (int l = 0; l < m->L; ++l) {
    std::string p = "blocks." + std::to_string(l) + ".";
    auto& b = m->blk[l];
    b.ln1_g = add(p + "ln1.g", C, 1);
    b.ln1_b = add(p + "ln1.b", C, 1);
    b.w_qkv = add(p + "attn.w_qkv", 3L * C, C);
    b.b_qkv = add(p + "attn.b_qkv", 3L * C, 1);
    b.w_o = add(p + "attn.w_o", C, C);
    b.b_o = add(p + "attn.b_o", C, 1);
    b.ln2_g = add(p + "ln2.g", C, 1);
    b.ln2_b = add(p + "ln2.b", C, 1);
    b.w_fc = add(p + "mlp.w_fc", F, C);
    b.b_fc = add(p + "mlp.b_fc", F, 1);
    b.w_proj = add(p + "mlp.w_proj", C, F);
    b.b_proj = add(p + "mlp.b_proj", C, 1);
  }
  m->o_lnf_g = add("lnf.g", C, 1);
  m->o_lnf_b = add("lnf.b", C, 1);
  m->o_head_w = m->o_head_b = -1;
  if (m->untied) {
    m->o_head_w = add("head.w", V, C, m->Vp * C);
    m->o_head_b = add("head.b", V, 1, std::max(m->Vp, m->ldz));
  }
}

std::vector<std::pair<const char*, GemmOp>> step_gemm_ops(lm_model* m);
GemmOp dw_op(const void* dY, long M, long N, const void* X, long K, float* dW);

// Token counts from which the blocks' weight gradients take the grouped
// launch (below, each GEMM's K is short enough that the per-GEMM K-split
// launches do as well)
constexpr long kDwGroupMinRows = 2048;
// backward_pass's return when the grouped launch's table could not be
// uploaded (a HIP error, not a shape the kernels reject)
constexpr int kTableUploadFailed = 2;

// Units of a grouped launch of every block's four weight gradients at M
// rows (-1: the grouped kernel does not take them).
long dw_group_units(lm_model* m, long M) {
  static const char dummy[256] = {0};
  const void* X = dummy;
  float* W = reinterpret_cast<float*>(const_cast<char*>(dummy));
  const long C = m->C, F = m->F;
  const GemmOp ops[4] = {dw_op(X, M, C, X, F, W), dw_op(X, M, F, X, C, W), dw_op(X, M, C, X, C, W),
                         dw_op(X, M, 3 * C, X, C, W)};
  std::vector<char> tab(gemm_group_table_bytes(4));
  int tn = 0;
  const int units = gemm_group_plan(ops, 4, tab.data(), &tn);
  return units < 0 ? -1 : (long)units * m->L;
}

// The vocabulary projection's weight gradient joins the blocks' grouped
// launch (as 128 x 192 units over the same K, appended after theirs) when
// that saves a whole round of the CUs: its units then fill the round the
// blocks' units leave partly empty, and its own launch (256 x 256 tiles, K
// split into slices) and split-K reduction go away. Measured on the
// GPT-2-small-shaped step (3456 + 1572 units: 20 rounds instead of 14 + 7).
// At the 32768-row workload the two would take as many rounds as apart
// (1536 + 384 units), so its head keeps the separate launch.
bool head_dw_grouped(lm_model* m, long M, const GemmOp& head) {
  const long blocks = dw_group_units(m, M);
  if (blocks < 0) return false;
  std::vector<char> tab(gemm_group_table_bytes(1));
  int tn = 0;
  const long units = gemm_group_plan(&head, 1, tab.data(), &tn);
  if (units < 0) return false;
  const long cus = gemm_cus();
  auto rounds = [&](long u) { return (u + cus - 1) / cus; };
  return rounds(blocks + units) < rounds(blocks) + rounds(units);
}

// K slices of the grouped launch's GEMMs: when its units (whole K each,
// the vocabulary projection's included where it joins) leave CUs idle, as
// many slices as fill them (at most 8); their partial sums are added in
// slice order by one reduction launch. Measured at 16384 rows of the
// 128-wide workload (107 units: 2 slices): the grouped weight gradients
// 0.191 -> 0.137 ms per step with the reduction; the wider workloads fill
// the CUs unsliced.
int dw_group_slices(lm_model* m) {
  const long M = m->M();
  long units = dw_group_units(m, M);
  if (units <= 0) return 1;
  static const char dummy[256] = {0};
  GemmOp head = dw_op(dummy, M, m->h16 ? m->Vp : m->V, dummy, m->C,
                      reinterpret_cast<float*>(const_cast<char*>(dummy)));
  head.lda = m->ldz;
  head.M_out = (int)m->V;
  if (head_dw_grouped(m, M, head)) {
    std::vector<char> tab(gemm_group_table_bytes(1));
    int tn = 0;
    units += gemm_group_plan(&head, 1, tab.data(), &tn);
  }
  return (int)std::max(1L, std::min(8L, (long)gemm_cus() / units));
}

// Lays out every slice of the arena (base == nullptr: size only).
void carve(lm_model* m, char* base) {
  Carver c{base};
  const long M = m->M(), C = m->C, F = m->F, L = m->L;
  const size_t A = m->act_size;
  m->params = c.take<float>(m->P);
  m->grads = c.take<float>(m->P);
  m->adam_m = c.take<float>(m->P);
  m->adam_v = c.take<float>(m->P);
  m->shadow = m->h16 ? c.take<uint16_t>(m->P) : nullptr;
  m->x = c.take<float>((L + 1) * M * C);
  m->xm = c.take<float>(L * M * C);
  m->y1 = c.take<char>(L * M * C * A);
  m->qkv = c.take<char>(L * M * 3 * C * A);
  m->o = c.take<char>(L * M * C * A);
  m->y2 = c.take<char>(L * M * C * A);
  m->gelu_d = c.take<char>(L * M * F * A);
  m->a = c.take<char>(L * M * F * A);
  m->hf = c.take<char>(M * C * A);
  m->logits = c.take<char>(M * m->ldz * A);
  m->mu1 = c.take<float>(L * M);
  m->r1 = c.take<float>(L * M);
  m->mu2 = c.take<float>(L * M);
  m->r2 = c.take<float>(L * M);
  m->muf = c.take<float>(M);
  m->rf = c.take<float>(M);
  m->lse = c.take<float>(L * M * m->H);
  m->g = c.take<float>(M * C);
  m->dy = c.take<float>(M * C);
  m->delta = c.take<float>(M * m->H);
  m->g_act = c.take<char>(M * C * A);
  m->dbig = c.take<char>(M * std::max(F, 3 * C) * A);
  m->dO = c.take<char>(M * C * A);
  if (m->dw_group) {
    m->g_act_l = c.take<char>(L * 2 * M * C * A);
    m->du_l = c.take<char>(L * M * F * A);
    m->dqkv_l = c.take<char>(L * M * 3 * C * A);
    m->dw_tab = c.take<char>(gemm_group_table_bytes(4 * (int)L + 1));  // + the vocabulary projection's
    if (m->dw_slices > 1)
      m->dw_part = c.take<float>((long)m->dw_slices * (L * (2 * C * F + 4 * C * C) + (long)(m->h16 ? m->Vp : m->V) * C));
  }
  long ln_blocks = (M + kLnRowsPerBlock - 1) / kLnRowsPerBlock;
  // partial sums of every LayerNorm of the backward (2 per block + the
  // final one), reduced together once the backward is done
  m->ln_part = c.take<float>((2 * L + 1) * 3 * ln_blocks * C);
  long col_blocks = (M + kColRows - 1) / kColRows;
  m->col_part = c.take<float>(col_blocks * std::max(std::max(F, 3 * C), m->untied ? m->ldz : 0L));
  // per-block partial column sums of every MLP-in and QKV bias gradient,
  // reduced together after the backward
  // (the MLP-in slot holds up to two partial rows per row block: those the
  // GELU' GEMM epilogue writes)
  m->bias_part = c.take<float>(L * col_blocks * (2 * F + 3 * C));
  // split-K partials of the GEMMs (at least what every GEMM of a step at
  // max_batch rows uses: with less, a GEMM runs unsplit); also the decode
  // attention's score scratch (max_batch * H * max_seq floats), which runs
  // between GEMMs
  m->gemm_ws_floats = std::max(8L * std::max(F, 3 * C) * std::max(F, C), (long)m->Bmax * m->H * m->S);
  for (auto& named : step_gemm_ops(m))
    m->gemm_ws_floats = std::max(m->gemm_ws_floats, gemm_ws_floats_needed(named.second, m->h16));
  m->gemm_ws = c.take<float>(m->gemm_ws_floats);
  for (int k = 0; k < 2; ++k) {
    EmbedBwdWs& e = k == 0 ? m->emb_tok : m->emb_pos;
    long nkeys = k == 0 ? m->V : m->S;
    e.counts = c.take<int32_t>(nkeys + 1);
    e.offsets = c.take<int32_t>(nkeys + 1);
    e.chunk_base = c.take<int32_t>(nkeys + 1);
    e.perm = c.take<int32_t>(M);
    e.rank_cap = csr_rank_ints((int)M, (int)nkeys);
    e.rank = c.take<int32_t>(e.rank_cap);
    e.partial = c.take<float>(embed_bwd_max_chunks((int)M, (int)nkeys) * C);
  }
  m->start = c.take<int32_t>(M);
  m->end = c.take<int32_t>(M);
  m->pos = c.take<int32_t>(M);
  m->n_valid = c.take<int32_t>(4);
  m->flags = c.take<uint32_t>(4);
  m->row_loss = c.take<float>(M);
  m->norm_scale = c.take<float>(4);
  m->stats_own = c.take<float>(4);
  m->scale_state = c.take<float>(2);
  m->norm_part = c.take<double>(kNormBlocks);
  m->bytes = align_up(c.off, kAlign);
}

lm_model* new_model(const lm_config* cfg) {
  lm_model* m = new lm_model();
  m->cfg = *cfg;
  m->V = cfg->vocab;
  m->C = cfg->d_model;
  m->H = cfg->n_heads;
  m->D = cfg->d_model / cfg->n_heads;
  m->F = cfg->d_mlp;
  m->L = cfg->n_layers;
  m->S = cfg->max_seq;
  m->Bmax = cfg->max_batch;
  m->prec = cfg->precision;
  m->h16 = m->prec != 0;
  m->untied = cfg->untied_head == 1;
  m->act_size = m->h16 ? 2 : 4;
  m->Vp = m->h16 ? round_up(m->V, 128) : m->V;
  m->ldz = m->h16 ? m->Vp : round_up(m->V, 4);
  build_table(m);
  m->dw_group = m->h16 && m->L > 0 && dw_group_units(m, m->M()) > 0;
  m->dw_slices = m->dw_group ? dw_group_slices(m) : 1;
  carve(m, nullptr);
  return m;
}

// --------------------------------------------------------------- launches
struct Launcher {
  lm_model* m;
  hipStream_t s;
  int cls = -1;
  Launcher(lm_model* m_, hipStream_t s_) : m(m_), s(s_) {}
  // bracket a group of launches of one kernel class with events
  template <typename F>
  void run(const char* name, double flops, double bytes, F&& f) {
    if (!m->prof.on) {
      f();
      return;
    }
    int c = m->prof.find(name);
    auto& cl = m->prof.cls[c];
    cl.launches += 1;
    cl.flops += flops;
    cl.bytes += bytes;
    hipEvent_t a = m->prof.take(), b = m->prof.take();
    (void)hipEventRecord(a, s);
    f();
    (void)hipEventRecord(b, s);
    m->prof.pending.push_back({c, a, b});
    if (m->prof.pending.size() > 4096) m->prof.drain();
  }
};

int gemm(lm_model* m, const GemmOp& op, hipStream_t s) {
  if (m->prec == 2) return gemm_f16(op, m->gemm_ws, m->gemm_ws_floats, s);
  if (m->prec == 1) return gemm_bf16(op, m->gemm_ws, m->gemm_ws_floats, s);
  return gemm_f32(op, m->gemm_ws, m->gemm_ws_floats, s);
}

// Y = X W^T (+ epilogue), X [M, K] activation, W [N, K] weight.
GemmOp fwd_op(lm_model* m, const void* X, long M, long K, long w_off, long N, void* Y, int epi) {
  GemmOp op;
  op.M = (int)M; op.N = (int)N; op.K = (int)K;
  op.A = X; op.lda = K; op.a_kc = true;
  op.B = m->W(w_off); op.ldb = K; op.b_kc = true;
  op.C = Y; op.ldc = N; op.epi = epi;
  return op;
}
// dX = dY W: dY [M, N] activation, W [N, K] -> dX [M, K]
GemmOp dx_op(lm_model* m, const void* dY, long M, long N, long w_off, long K, void* dX, int epi) {
  GemmOp op;
  op.M = (int)M; op.N = (int)K; op.K = (int)N;
  op.A = dY; op.lda = N; op.a_kc = true;
  op.B = m->W(w_off); op.ldb = K; op.b_kc = false;
  op.C = dX; op.ldc = K; op.epi = epi;
  return op;
}
// dW = dY^T X: dY [M, N], X [M, K] -> dW [N, K] fp32 (overwritten)
GemmOp dw_op(const void* dY, long M, long N, const void* X, long K, float* dW) {
  GemmOp op;
  op.M = (int)N; op.N = (int)K; op.K = (int)M;
  op.A = dY; op.lda = N; op.a_kc = false;
  op.B = X; op.ldb = K; op.b_kc = false;
  op.C = dW; op.ldc = K; op.epi = EPI_STORE; op.c_f32 = true;
  return op;
}

// Vocabulary projection z = h_f W^T (+ b): W = wte (tied) or head.w with the
// bias head.b (untied). bf16: N = Vp; the padding rows of W are zero, so the
// padding columns of z are too (plus the zero padding of the bias).
GemmOp head_op(lm_model* m, const void* hf, long M, void* z) {
  GemmOp op = fwd_op(m, hf, M, m->C, m->head_w(), m->h16 ? m->Vp : m->V, z, EPI_STORE);
  op.ldc = m->ldz;
  if (m->untied) op.bias = m->P_(m->o_head_b);
  return op;
}

// Every GEMM a step launches, built as the passes build them for the largest
// batch the model accepts (M = max_batch * max_seq); the operand pointers
// are placeholders (only shapes, layouts and epilogues matter to the
// dispatcher's rules and to the split-K workspace).
std::vector<std::pair<const char*, GemmOp>> step_gemm_ops(lm_model* m) {
  static const char dummy[256] = {0};
  void* X = const_cast<char*>(dummy);
  const float* R = reinterpret_cast<const float*>(dummy);
  const long M = m->M(), C = m->C, F = m->F;
  const long Vh = m->h16 ? m->Vp : m->V;
  const lm_model::Blk b{};
  std::vector<std::pair<const char*, GemmOp>> ops;
  {
    GemmOp op = fwd_op(m, X, M, C, b.w_qkv, 3 * C, X, EPI_STORE);
    op.bias = R;
    ops.push_back({"QKV projection", op});
    op = fwd_op(m, X, M, C, b.w_o, C, X, EPI_RESID);
    op.bias = R; op.R = R; op.ldr = C;
    ops.push_back({"attention output", op});
    op = fwd_op(m, X, M, C, b.w_fc, F, X, EPI_GELU);
    op.bias = R; op.aux = X; op.ld_aux = F;
    ops.push_back({"MLP in", op});
    op = fwd_op(m, X, M, F, b.w_proj, C, X, EPI_RESID);
    op.bias = R; op.R = R; op.ldr = C;
    ops.push_back({"MLP out", op});
    ops.push_back({"vocabulary projection", head_op(m, X, M, X)});
    op = dw_op(X, M, Vh, X, C, const_cast<float*>(R));
    op.lda = m->ldz; op.M_out = m->V;
    ops.push_back({"vocabulary weight gradient", op});
    op = dx_op(m, X, M, Vh, 0, C, X, EPI_STORE);
    op.lda = m->ldz; op.c_f32 = true;
    ops.push_back({"vocabulary input gradient", op});
    ops.push_back({"MLP-out weight gradient", dw_op(X, M, C, X, F, const_cast<float*>(R))});
    op = dx_op(m, X, M, C, 0, F, X, EPI_DGELU);
    op.aux = X; op.ld_aux = F;
    ops.push_back({"MLP-out input gradient", op});
    ops.push_back({"MLP-in weight gradient", dw_op(X, M, F, X, C, const_cast<float*>(R))});
    op = dx_op(m, X, M, F, 0, C, X, EPI_STORE);
    op.c_f32 = true;
    ops.push_back({"MLP-in input gradient", op});
    ops.push_back({"attention-output weight gradient", dw_op(X, M, C, X, C, const_cast<float*>(R))});
    ops.push_back({"attention-output input gradient", dx_op(m, X, M, C, 0, C, X, EPI_STORE)});
    ops.push_back({"QKV weight gradient", dw_op(X, M, 3 * C, X, C, const_cast<float*>(R))});
    op = dx_op(m, X, M, 3 * C, 0, C, X, EPI_STORE);
    op.c_f32 = true;
    ops.push_back({"QKV input gradient", op});
  }
  return ops;
}

// The step's GEMMs checked against the dispatcher's rules without launching
// anything. The rules depend on the row count only through the bytes an
// operand spans, which grow with it, so every smaller batch passes too: a
// step can then never stop part-way through its launches on a rejected shape.
lm_status check_model_shapes(lm_model* m) {
  const long M = m->M();
  const auto ops = step_gemm_ops(m);
  for (auto& [what, op] : ops)
    if (gemm_check(op, m->h16))
      return fail(LM_ERR_UNSUPPORTED, std::string("the ") + what + " GEMM breaks the kernels' limits at " +
                                          "max_batch * max_seq = " + std::to_string(M) +
                                          " rows (each 16-bit operand must span less than 2 GiB)");
  return LM_OK;
}

// Runs f(tag) with a null pointer of the model's activation type (float,
// bf16 or f16) as the tag.
template <typename F>
int with_act(const lm_model* m, F&& f) {
  if (m->prec == 2) return f(static_cast<f16*>(nullptr));
  if (m->prec == 1) return f(static_cast<bf16*>(nullptr));
  return f(static_cast<float*>(nullptr));
}

template <typename E>
int forward_pass(lm_model* m, Launcher& Lr, const int32_t* tok, const int32_t* doc, int B, int T) {
  hipStream_t s = Lr.s;
  const long M = (long)B * T, C = m->C, F = m->F, H = m->H;
  const double Mf = (double)M, A = (double)sizeof(E);
  int rc = 0;
  Lr.run("index_layout", 0, 12.0 * M, [&] { launch_index_layout(doc, B, T, m->start, m->end, m->pos, m->flags, s); });
  Lr.run("embed_fwd", 0, Mf * C * 12.0, [&] {
    launch_embed_fwd(tok, m->pos, m->params + m->o_wte, m->params + m->o_wpe, (int)M, (int)C, m->V, m->x, m->flags, s);
  });
  AttnArgs at{};
  at.start = m->start; at.end = m->end; at.B = B; at.T = T; at.H = (int)H; at.D = m->D;
  for (int l = 0; l < m->L; ++l) {
    const auto& b = m->blk[l];
    float* xl = m->x + l * M * C;
    float* xml = m->xm + l * M * C;
    E* y1 = m->act<E>(m->y1, l * M * C);
    E* qkv = m->act<E>(m->qkv, l * M * 3 * C);
    E* o = m->act<E>(m->o, l * M * C);
    E* y2 = m->act<E>(m->y2, l * M * C);
    E* gd = m->act<E>(m->gelu_d, l * M * F);
    E* a = m->act<E>(m->a, l * M * F);
    Lr.run("layernorm_fwd", 0, Mf * C * (4 + A), [&] {
      launch_ln_fwd<E>(xl, m->P_(b.ln1_g), m->P_(b.ln1_b), (int)M, (int)C, m->cfg.ln_eps, y1, m->mu1 + l * M,
                       m->r1 + l * M, s);
    });
    {
      GemmOp op = fwd_op(m, y1, M, C, b.w_qkv, 3 * C, qkv, EPI_STORE);
      op.bias = m->P_(b.b_qkv);
      Lr.run("gemm_qkv_fwd", 2.0 * M * 3 * C * C, 0, [&] { rc |= gemm(m, op, s); });
    }
    at.qkv = qkv; at.o = o; at.lse = m->lse + l * M * H;
    Lr.run("attn_fwd", 0, 0, [&] {
      if constexpr (std::is_same_v<E, float>) rc |= attn_fwd_f32(at, s);
      else rc |= attn_fwd16<E>(at, s);
    });
    {
      GemmOp op = fwd_op(m, o, M, C, b.w_o, C, xml, EPI_RESID);
      op.bias = m->P_(b.b_o); op.R = xl; op.ldr = C;
      Lr.run("gemm_attnout_fwd", 2.0 * M * C * C, 0, [&] { rc |= gemm(m, op, s); });
    }
    Lr.run("layernorm_fwd", 0, Mf * C * (4 + A), [&] {
      launch_ln_fwd<E>(xml, m->P_(b.ln2_g), m->P_(b.ln2_b), (int)M, (int)C, m->cfg.ln_eps, y2, m->mu2 + l * M,
                       m->r2 + l * M, s);
    });
    {
      GemmOp op = fwd_op(m, y2, M, C, b.w_fc, F, gd, EPI_GELU);
      op.bias = m->P_(b.b_fc); op.aux = a; op.ld_aux = F;
      Lr.run("gemm_fc1_fwd", 2.0 * M * F * C, 0, [&] { rc |= gemm(m, op, s); });
    }
    {
      GemmOp op = fwd_op(m, a, M, F, b.w_proj, C, m->x + (l + 1) * M * C, EPI_RESID);
      op.bias = m->P_(b.b_proj); op.R = xml; op.ldr = C;
      Lr.run("gemm_fc2_fwd", 2.0 * M * C * F, 0, [&] { rc |= gemm(m, op, s); });
    }
  }
  E* hf = m->act<E>(m->hf, 0);
  Lr.run("layernorm_fwd", 0, Mf * C * (4 + A), [&] {
    launch_ln_fwd<E>(m->x + m->L * M * C, m->P_(m->o_lnf_g), m->P_(m->o_lnf_b), (int)M, (int)C, m->cfg.ln_eps, hf,
                     m->muf, m->rf, s);
  });
  {
    GemmOp op = head_op(m, hf, M, m->act<E>(m->logits, 0));
    Lr.run("gemm_head_fwd", 2.0 * M * m->V * C, 0, [&] { rc |= gemm(m, op, s); });
  }
  return rc;
}

// One generation step with a key/value cache: B new tokens, all at position
// pos, run through every block with M = B rows; each block appends its keys
// and values at pos and attends over cache positions 0 .. pos; the head
// writes B rows of logits. Same kernels and epilogues as the forward pass.
// d_pos (nullable): the position in device memory instead of pos, read by
// the kernels when they run (clamped to [1, max_seq - 1]).
template <typename E>
int decode_pass(lm_model* m, Launcher& Lr, const int32_t* tok, int B, int pos, E* cache,
                const int32_t* d_pos = nullptr) {
  hipStream_t s = Lr.s;
  const long M = B, C = m->C, F = m->F, H = m->H, S = m->S;
  const double Mf = (double)M, A = (double)sizeof(E);
  int rc = 0;
  if (d_pos) launch_fill_pos(m->pos, d_pos, (int)S, M, s);
  else launch_fill_u32(reinterpret_cast<uint32_t*>(m->pos), (uint32_t)pos, M, s);
  Lr.run("embed_fwd", 0, Mf * C * 12.0, [&] {
    launch_embed_fwd(tok, m->pos, m->params + m->o_wte, m->params + m->o_wpe, (int)M, (int)C, m->V, m->x, m->flags, s);
  });
  for (int l = 0; l < m->L; ++l) {
    const auto& b = m->blk[l];
    float* xl = m->x + l * M * C;
    float* xml = m->xm + l * M * C;
    E* y1 = m->act<E>(m->y1, l * M * C);
    E* qkv = m->act<E>(m->qkv, l * M * 3 * C);
    E* o = m->act<E>(m->o, l * M * C);
    E* y2 = m->act<E>(m->y2, l * M * C);
    E* gd = m->act<E>(m->gelu_d, l * M * F);
    E* a = m->act<E>(m->a, l * M * F);
    E* kc = cache + 2L * l * B * S * C;
    E* vc = kc + (long)B * S * C;
    Lr.run("layernorm_fwd", 0, Mf * C * (4 + A), [&] {
      launch_ln_fwd<E>(xl, m->P_(b.ln1_g), m->P_(b.ln1_b), (int)M, (int)C, m->cfg.ln_eps, y1, m->mu1 + l * M,
                       m->r1 + l * M, s);
    });
    {
      GemmOp op = fwd_op(m, y1, M, C, b.w_qkv, 3 * C, qkv, EPI_STORE);
      op.bias = m->P_(b.b_qkv);
      Lr.run("gemm_qkv_fwd", 2.0 * M * 3 * C * C, 0, [&] { rc |= gemm(m, op, s); });
    }
    Lr.run("attn_decode", 0, 0, [&] {
      launch_kv_store<E>(qkv, B, 1, (int)C, (int)S, pos, kc, vc, s, d_pos);
      rc |= launch_attn_decode<E>(qkv, kc, vc, B, (int)H, m->D, (int)S, pos + 1, o, m->gemm_ws, s, d_pos);
    });
    {
      GemmOp op = fwd_op(m, o, M, C, b.w_o, C, xml, EPI_RESID);
      op.bias = m->P_(b.b_o); op.R = xl; op.ldr = C;
      Lr.run("gemm_attnout_fwd", 2.0 * M * C * C, 0, [&] { rc |= gemm(m, op, s); });
    }
    Lr.run("layernorm_fwd", 0, Mf * C * (4 + A), [&] {
      launch_ln_fwd<E>(xml, m->P_(b.ln2_g), m->P_(b.ln2_b), (int)M, (int)C, m->cfg.ln_eps, y2, m->mu2 + l * M,
                       m->r2 + l * M, s);
    });
    {
      GemmOp op = fwd_op(m, y2, M, C, b.w_fc, F, gd, EPI_GELU);
      op.bias = m->P_(b.b_fc); op.aux = a; op.ld_aux = F;
      Lr.run("gemm_fc1_fwd", 2.0 * M * F * C, 0, [&] { rc |= gemm(m, op, s); });
    }
    {
      GemmOp op = fwd_op(m, a, M, F, b.w_proj, C, m->x + (l + 1) * M * C, EPI_RESID);
      op.bias = m->P_(b.b_proj); op.R = xml; op.ldr = C;
      Lr.run("gemm_fc2_fwd", 2.0 * M * C * F, 0, [&] { rc |= gemm(m, op, s); });
    }
  }
  E* hf = m->act<E>(m->hf, 0);
  Lr.run("layernorm_fwd", 0, Mf * C * (4 + A), [&] {
    launch_ln_fwd<E>(m->x + m->L * M * C, m->P_(m->o_lnf_g), m->P_(m->o_lnf_b), (int)M, (int)C, m->cfg.ln_eps, hf,
                     m->muf, m->rf, s);
  });
  {
    GemmOp op = head_op(m, hf, M, m->act<E>(m->logits, 0));
    Lr.run("gemm_head_fwd", 2.0 * M * m->V * C, 0, [&] { rc |= gemm(m, op, s); });
  }
  return rc;
}

template <typename E>
int backward_pass(lm_model* m, Launcher& Lr, const int32_t* tok, const int32_t* tgt, int B, int T, float* stats,
                  bool packed) {
  hipStream_t s = Lr.s;
  const long M = (long)B * T, C = m->C, F = m->F, H = m->H, V = m->V;
  const double Mf = (double)M, A = (double)sizeof(E);
  int rc = 0;
  E* z = m->act<E>(m->logits, 0);
  Lr.run("count_valid", 0, 4.0 * M, [&] { launch_count_valid(tgt, (int)M, m->V, m->n_valid, stats, m->flags, s); });
  Lr.run("xent", 0, Mf * V * 2 * A, [&] {
    launch_xent<E>(z, m->ldz, (int)M, m->V, tgt, m->n_valid, m->row_loss, m->scaler().state, s);
  });
  Lr.run("loss_reduce", 0, 4.0 * M, [&] { launch_loss_reduce(m->row_loss, (int)M, m->n_valid, stats, s); });
  E* hf = m->act<E>(m->hf, 0);
  E* g_act = m->act<E>(m->g_act, 0);
  // head: dW = dz^T h_f (tied: the first writer of the wte gradient); dh_f =
  // dz W; untied: the bias gradient is the column sums of dz (its zero
  // padding columns give the zero padding of the bias gradient)
  // the weight gradients of the blocks: one grouped launch after the loop
  // (reading per-layer copies of the output gradients), or each right away;
  // the head's joins that launch where it saves a round (z and h_f stay
  // untouched until then)
  const bool grouped = m->dw_group && M >= kDwGroupMinRows;
  GemmOp head_dw = dw_op(z, M, m->h16 ? m->Vp : V, hf, C, m->grads + m->head_w());
  head_dw.lda = m->ldz;
  head_dw.M_out = (int)V;
  const bool head_in_group = grouped && head_dw_grouped(m, M, head_dw);
  if (!head_in_group) Lr.run("gemm_head_bwd_dw", 2.0 * M * V * C, 0, [&] { rc |= gemm(m, head_dw, s); });
  if (m->untied)
    Lr.run("bias_grad", 0, Mf * m->ldz * A, [&] {
      launch_colsum<E>(z, m->ldz, (int)M, (int)m->ldz, m->col_part, m->grads + m->o_head_b, s);
    });
  {
    GemmOp op = dx_op(m, z, M, m->h16 ? m->Vp : V, m->head_w(), C, m->dy, EPI_STORE);
    op.lda = m->ldz;
    op.c_f32 = true;
    Lr.run("gemm_head_bwd_dx", 2.0 * M * V * C, 0, [&] { rc |= gemm(m, op, s); });
  }
  long ln_blocks = (M + kLnRowsPerBlock - 1) / kLnRowsPerBlock;
  // LayerNorm backward; the column sums of its output gradient g are the
  // gradient of the bias added to the residual stream right before the
  // LayerNorm's input (b_proj of the block below for ln_1 and ln_f, b_o of
  // the same block for ln_2), so they come out of the same pass (dcol). Each
  // LayerNorm writes its per-block partial sums into a slot of its own; all
  // slots are reduced in one launch after the backward (the sums are only
  // read by the optimizer).
  // (one descriptor per LayerNorm, 2L + 1 of them; launched kColsumBatch at
  // a time)
  struct LnPart {
    const float *pa, *pb, *pc;
    float *oa, *ob, *oc;
  };
  std::vector<LnPart> lnb;
  const long col_blocks = (M + kColRows - 1) / kColRows;
  auto fc_part = [&](int l) { return m->bias_part + (long)l * col_blocks * (2 * F + 3 * C); };
  auto qkv_part = [&](int l) { return fc_part(l) + 2 * col_blocks * F; };
  // the MLP-in bias gradient's partial sums come from the GELU' GEMM's
  // epilogue where its kernel writes them (fc_rows rows), else from a column
  // sum over its output (col_blocks rows)
  long fc_rows = col_blocks;
  bool fc_fused = false;
  if (m->prec != 0) {
    GemmOp probe = dx_op(m, m->g_act, M, C, 0, F, m->dbig, EPI_DGELU);
    probe.aux = m->dbig; probe.ld_aux = F;
    const int rows = gemm16_colsum_rows(probe);
    if (rows > 0 && rows <= 2 * col_blocks) {
      fc_fused = true;
      fc_rows = rows;
    }
  }
  std::vector<float*> fc_pa(m->L), fc_oa(m->L), qkv_pa(m->L), qkv_oa(m->L);
  struct { std::vector<float*>& pa; std::vector<float*>& oa; } fcb{fc_pa, fc_oa}, qkvb{qkv_pa, qkv_oa};
  double ln_red_bytes = 0;
  std::vector<GemmOp> dw_ops;
  std::vector<std::pair<const E*, float*>> qkv_colsum;
  const bool batch_qkv_colsum = grouped && M * 3 * C * (long)sizeof(E) <= (64L << 20);
  auto weight_grad = [&](const char* name, GemmOp op) {
    if (grouped) dw_ops.push_back(op);
    else Lr.run(name, 2.0 * op.M * op.N * op.K, 0, [&] { rc |= gemm(m, op, s); });
  };
  // the 16-bit output gradient of block l's MLP (k = 0) or attention (k = 1)
  // output, which a LayerNorm backward writes
  auto g_act_of = [&](int l, int k) -> E* {
    return grouped && l >= 0 ? m->act<E>(m->g_act_l, ((long)l * 2 + k) * M * C) : g_act;
  };
  auto ln_bwd = [&](const float* x, const float* mu, const float* r, long g_off, long b_off, const float* g_in,
                    float* dcol, E* g_out) {
    float* pdg = m->ln_part + (long)lnb.size() * 3 * ln_blocks * C;
    float* pdb = pdg + ln_blocks * C;
    float* pdc = pdg + 2 * ln_blocks * C;
    Lr.run("layernorm_bwd", 0, Mf * C * ((g_in ? 4 * 4 : 3 * 4) + A), [&] {
      launch_ln_bwd<E>(m->dy, x, mu, r, m->P_(g_off), (int)M, (int)C, g_in, m->g, g_out, pdg, pdb,
                       dcol ? pdc : nullptr, s);
    });
    lnb.push_back({pdg, pdb, dcol ? pdc : nullptr, m->grads + g_off, m->grads + b_off, dcol});
    ln_red_bytes += (dcol ? 3.0 : 2.0) * ln_blocks * C * 4;
  };
  // the collected reductions, kColsumBatch per launch
  auto ln_reduce = [&] {
    const int n_ln = (int)lnb.size();
    for (int i0 = 0; i0 < n_ln; i0 += kColsumBatch) {
      ColsumBatch part{};
      const int n = std::min(kColsumBatch, n_ln - i0);
      for (int i = 0; i < n; ++i) {
        const LnPart& d = lnb[i0 + i];
        part.pa[i] = d.pa; part.pb[i] = d.pb; part.pc[i] = d.pc;
        part.oa[i] = d.oa; part.ob[i] = d.ob; part.oc[i] = d.oc;
      }
      launch_colsum_partials_batch(part, n, (int)ln_blocks, (int)C, s);
    }
  };
  // (with no blocks the final LayerNorm reads the embeddings: no bias below it)
  ln_bwd(m->x + m->L * M * C, m->muf, m->rf, m->o_lnf_g, m->o_lnf_b, nullptr,
         m->L > 0 ? m->grads + m->blk[m->L - 1].b_proj : nullptr, g_act_of(m->L - 1, 0));
  E* dO = m->act<E>(m->dO, 0);
  for (int l = m->L - 1; l >= 0; --l) {
    const auto& b = m->blk[l];
    E* g_mlp = g_act_of(l, 0);
    E* g_att = g_act_of(l, 1);
    E* du = grouped ? m->act<E>(m->du_l, l * M * F) : m->act<E>(m->dbig, 0);
    E* dqkv = grouped ? m->act<E>(m->dqkv_l, l * M * 3 * C) : m->act<E>(m->dbig, 0);
    float* xl = m->x + l * M * C;
    float* xml = m->xm + l * M * C;
    E* y1 = m->act<E>(m->y1, l * M * C);
    E* qkv = m->act<E>(m->qkv, l * M * 3 * C);
    E* o = m->act<E>(m->o, l * M * C);
    E* y2 = m->act<E>(m->y2, l * M * C);
    E* gd = m->act<E>(m->gelu_d, l * M * F);
    E* a = m->act<E>(m->a, l * M * F);
    // MLP out: x_{l+1} = xm + a W_proj^T + b_proj
    weight_grad("gemm_fc2_bwd_dw", dw_op(g_mlp, M, C, a, F, m->grads + b.w_proj));
    {
      GemmOp op = dx_op(m, g_mlp, M, C, b.w_proj, F, du, EPI_DGELU);
      op.aux = gd; op.ld_aux = F;
      if (fc_fused) op.colsum = fc_part(l);
      Lr.run("gemm_fc2_bwd_dx", 2.0 * M * C * F, 0, [&] { rc |= gemm(m, op, s); });
    }
    // MLP in: u = y2 W_fc^T + b_fc
    weight_grad("gemm_fc1_bwd_dw", dw_op(du, M, F, y2, C, m->grads + b.w_fc));
    if (!fc_fused)
      Lr.run("bias_grad", 0, Mf * F * A, [&] { launch_colsum_stage1<E>(du, F, (int)M, (int)F, fc_part(l), s); });
    fcb.pa[l] = fc_part(l);
    fcb.oa[l] = m->grads + b.b_fc;
    {
      GemmOp op = dx_op(m, du, M, F, b.w_fc, C, m->dy, EPI_STORE);
      op.c_f32 = true;
      Lr.run("gemm_fc1_bwd_dx", 2.0 * M * C * F, 0, [&] { rc |= gemm(m, op, s); });
    }
    ln_bwd(xml, m->mu2 + l * M, m->r2 + l * M, b.ln2_g, b.ln2_b, m->g, m->grads + b.b_o, g_att);
    // attention out: xm = x + o W_o^T + b_o
    weight_grad("gemm_attnout_bwd_dw", dw_op(g_att, M, C, o, C, m->grads + b.w_o));
    Lr.run("gemm_attnout_bwd_dx", 2.0 * M * C * C, 0, [&] { rc |= gemm(m, dx_op(m, g_att, M, C, b.w_o, C, dO, EPI_STORE), s); });
    {
      AttnArgs at{};
      at.qkv = qkv; at.start = m->start; at.end = m->end; at.B = B; at.T = T; at.H = (int)H; at.D = m->D;
      at.o = o; at.lse = m->lse + l * M * H; at.dout = dO; at.delta = m->delta; at.dqkv = dqkv;
      static const char* names[3] = {"attn_bwd_delta", "attn_bwd_dq", "attn_bwd_dkv"};
      // bf16: the dQ pass computes delta itself (part 0 launches nothing)
      for (int part = m->h16 ? 1 : 0; part < 3; ++part)
        Lr.run(names[part], 0, part == 0 ? Mf * C * 2 * A : 0, [&] {
          if constexpr (std::is_same_v<E, float>) rc |= attn_bwd_part_f32(at, part, s);
          else rc |= attn_bwd_part16<E>(at, part, s);
        });
    }
    weight_grad("gemm_qkv_bwd_dw", dw_op(dqkv, M, 3 * C, y1, C, m->grads + b.w_qkv));
    // (grouped: every layer's dqkv is kept until after the loop; up to 64 MB
    // each, their column sums go out in one launch there. Measured: at 8192 x
    // 2304 (37.7 MB) 12 such launches took 0.118 ms per step, the batched one
    // 0.099; at 32768 x 1536 (100 MB, no longer in the caches once the loop
    // is done) 8 took 0.163 ms, the batched one 0.180)
    if (batch_qkv_colsum) qkv_colsum.push_back({dqkv, qkv_part(l)});
    else Lr.run("bias_grad", 0, Mf * 3 * C * A, [&] { launch_colsum_stage1<E>(dqkv, 3 * C, (int)M, (int)(3 * C), qkv_part(l), s); });
    qkvb.pa[l] = qkv_part(l);
    qkvb.oa[l] = m->grads + b.b_qkv;
    {
      GemmOp op = dx_op(m, dqkv, M, 3 * C, b.w_qkv, C, m->dy, EPI_STORE);
      op.c_f32 = true;
      Lr.run("gemm_qkv_bwd_dx", 2.0 * M * 3 * C * C, 0, [&] { rc |= gemm(m, op, s); });
    }
    ln_bwd(xl, m->mu1 + l * M, m->r1 + l * M, b.ln1_g, b.ln1_b, m->g, l > 0 ? m->grads + m->blk[l - 1].b_proj : nullptr,
           g_act_of(l - 1, 0));
  }
  if constexpr (sizeof(E) == 2) {
    if (!qkv_colsum.empty())
      Lr.run("bias_grad", 0, Mf * 3 * C * A * (double)qkv_colsum.size(), [&] {
        for (size_t i0 = 0; i0 < qkv_colsum.size(); i0 += kColsumBatch) {
          Colsum16Batch bt{};
          const int n = (int)std::min((size_t)kColsumBatch, qkv_colsum.size() - i0);
          for (int i = 0; i < n; ++i) {
            bt.a[i] = qkv_colsum[i0 + i].first;
            bt.part[i] = qkv_colsum[i0 + i].second;
          }
          launch_colsum_stage1_batch<E>(bt, n, 3 * C, (int)M, (int)(3 * C), s);
        }
      });
  }
  if (grouped) {
    if (head_in_group) dw_ops.push_back(head_dw);
    // K slices (each at least 512 of the M token rows) into the partial-sum
    // buffer, laid out op after op
    const int slices = (int)std::min((long)m->dw_slices, std::max(1L, M / 512));
    std::vector<float*> part(dw_ops.size(), nullptr);
    if (slices > 1) {
      float* p = m->dw_part;
      for (size_t i = 0; i < dw_ops.size(); ++i) {
        dw_ops[i].force_split = slices;
        part[i] = p;
        p += (long)slices * dw_ops[i].M * dw_ops[i].N;
      }
    }
    // the table depends on the token count (the K of these GEMMs): uploaded
    // when it differs from the last upload, after the stream has drained (the
    // previous launch may still read the device copy)
    std::vector<char> tab(gemm_group_table_bytes((int)dw_ops.size()));
    int tn = 0;
    const int units = gemm_group_plan(dw_ops.data(), (int)dw_ops.size(), tab.data(), &tn, part.data());
    double flops = 0;
    for (const GemmOp& op : dw_ops) flops += 2.0 * (op.M_out > 0 ? op.M_out : op.M) * op.N * op.K;
    if (units < 0) return -1;
    if (tab != m->dw_tab_host) {
      if (hipStreamSynchronize(s) != hipSuccess ||
          hipMemcpy(m->dw_tab, tab.data(), tab.size(), hipMemcpyHostToDevice) != hipSuccess)
        return kTableUploadFailed;
      m->dw_tab_host = tab;
    }
    Lr.run("gemm_dw_group", flops, 0, [&] {
      rc |= gemm_group_launch(m->prec == 2, tn, m->dw_tab, units, s);
      if (slices > 1)
        for (size_t i0 = 0; i0 < dw_ops.size(); i0 += kGroupReduceMax) {
          GroupReduce gr{};
          gr.n = (int)std::min((size_t)kGroupReduceMax, dw_ops.size() - i0);
          for (int i = 0; i < gr.n; ++i) {
            const GemmOp& op = dw_ops[i0 + i];
            gr.part[i] = part[i0 + i];
            gr.dst[i] = static_cast<float*>(op.C);
            gr.rows[i] = op.M_out > 0 ? op.M_out : op.M;
            gr.cols[i] = op.N;
            gr.ldc[i] = op.ldc;
            gr.S[i] = gemm_group_slices_of(op);
            gr.stride[i] = (long)op.M * op.N;
          }
          launch_group_reduce(gr, s);
        }
    });
  }
  // embedding: dwte[tok] += dx0 (on top of the tied head's part, else from
  // zero), dwpe[pos] = sum dx0
  Lr.run("layernorm_bwd_reduce", 0, ln_red_bytes, ln_reduce);
  // the MLP-in and QKV bias gradients from their partial sums, in batches
  Lr.run("bias_grad_reduce", 0, 4.0 * (fc_rows * F + col_blocks * 3 * C) * m->L, [&] {
    for (int l0 = 0; l0 < m->L; l0 += kColsumBatch) {
      const int n = std::min(kColsumBatch, m->L - l0);
      ColsumBatch f{}, q{};
      for (int i = 0; i < n; ++i) {
        f.pa[i] = fcb.pa[l0 + i]; f.oa[i] = fcb.oa[l0 + i];
        q.pa[i] = qkvb.pa[l0 + i]; q.oa[i] = qkvb.oa[l0 + i];
      }
      launch_colsum_partials_batch(f, n, (int)fc_rows, (int)F, s);
      launch_colsum_partials_batch(q, n, (int)col_blocks, (int)(3 * C), s);
    }
  });
  Lr.run("embed_bwd", 0, Mf * C * 8, [&] {
    launch_csr(tok, (int)M, m->V, m->emb_tok, s);
    launch_segment_sum(m->g, tok, (int)M, (int)C, m->V, m->emb_tok, m->grads + m->o_wte, !m->untied, s);
    // without packed documents row b T + t has position t: a column sum over
    // the batch, with no sort
    if (packed) {
      launch_csr(m->pos, (int)M, m->S, m->emb_pos, s);
      launch_segment_sum(m->g, m->pos, (int)M, (int)C, m->S, m->emb_pos, m->grads + m->o_wpe, false, s);
    } else {
      launch_pos_colsum(m->g, B, T, (int)C, m->S, m->grads + m->o_wpe, s);
    }
  });
  return rc;
}

lm_status check_batch(lm_model* m, int B, int T) {
  if (B < 1 || T < 1) return fail(LM_ERR_SHAPE, "B and T must be >= 1");
  if (B > m->Bmax) return fail(LM_ERR_SHAPE, "B exceeds max_batch");
  if (T > m->S) return fail(LM_ERR_SHAPE, "T exceeds max_seq");
  return LM_OK;
}

lm_status hip_status(const char* what) {
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(LM_ERR_HIP, std::string(what) + ": " + hipGetErrorString(e));
  return LM_OK;
}

}  // namespace

extern "C" {

size_t lm_workspace_bytes(const lm_config* cfg) {
  if (validate(cfg) != LM_OK) return 0;
  lm_model* m = new_model(cfg);
  size_t b = check_model_shapes(m) == LM_OK ? m->bytes : 0;
  delete m;
  return b;
}

lm_status model_create(const lm_config* cfg, void* d_arena, size_t arena_bytes, void* stream, lm_model** out) {
  if (!out) return fail(LM_ERR_ARG, "out is NULL");
  *out = nullptr;
  lm_status st = validate(cfg);
  if (st != LM_OK) return st;
  if (!d_arena) return fail(LM_ERR_ARG, "arena is NULL");
  if (reinterpret_cast<uintptr_t>(d_arena) % kAlign) return fail(LM_ERR_WORKSPACE, "arena must be 256-byte aligned");
  lm_model* m = new_model(cfg);
  if ((st = check_model_shapes(m)) != LM_OK) {
    delete m;
    return st;
  }
  if (arena_bytes < m->bytes) {
    size_t need = m->bytes;
    delete m;
    return fail(LM_ERR_WORKSPACE, "arena too small: need " + std::to_string(need) + " bytes");
  }
  carve(m, reinterpret_cast<char*>(d_arena));
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  // zero parameters, gradients, moments and the bf16 copy (one contiguous run)
  char* z0 = reinterpret_cast<char*>(m->params);
  char* z1 = m->shadow ? reinterpret_cast<char*>(m->shadow + m->P) : reinterpret_cast<char*>(m->adam_v + m->P);
  launch_fill_u32(reinterpret_cast<uint32_t*>(z0), 0u, (long)((z1 - z0) / 4), s);
  launch_fill_u32(m->flags, 0u, 4, s);
  if (m->prec == 2) {
    // the default dynamic loss scale: S = 2^16, no finite steps yet
    const float init[2] = {65536.f, 0.f};
    uint32_t bits[2];
    std::memcpy(bits, init, sizeof(bits));
    launch_fill_u32(reinterpret_cast<uint32_t*>(m->scale_state), bits[0], 1, s);
    launch_fill_u32(reinterpret_cast<uint32_t*>(m->scale_state) + 1, bits[1], 1, s);
  }
  st = hip_status("model_create");
  if (st != LM_OK) {
    delete m;
    return st;
  }
  *out = m;
  return LM_OK;
}

void model_destroy(lm_model* m) { delete m; }

lm_status model_config(const lm_model* m, lm_config* out) {
  if (!m || !out) return fail(LM_ERR_ARG, "model or out is NULL");
  *out = m->cfg;
  return LM_OK;
}

lm_status model_param_table(const lm_model* m, lm_tensor_info* out, int32_t* count, int64_t* total) {
  if (!m || !count) return fail(LM_ERR_ARG, "model or count is NULL");
  int32_t cap = *count;
  if (out) {
    for (int32_t i = 0; i < cap && i < (int32_t)m->table.size(); ++i) {
      std::memset(out[i].name, 0, sizeof(out[i].name));
      std::strncpy(out[i].name, m->table[i].name.c_str(), sizeof(out[i].name) - 1);
      out[i].offset = m->table[i].off;
      out[i].rows = m->table[i].rows;
      out[i].cols = m->table[i].cols;
    }
  }
  *count = (int32_t)m->table.size();
  if (total) *total = m->P;
  return LM_OK;
}

static float* buf_of(const lm_model* m, lm_buf which) {
  switch (which) {
    case LM_PARAMS: return m->params;
    case LM_GRADS: return m->grads;
    case LM_ADAM_M: return m->adam_m;
    case LM_ADAM_V: return m->adam_v;
  }
  return nullptr;
}

lm_status model_set(lm_model* m, lm_buf which, const float* src, int src_on_device, void* stream) {
  if (!m || !src) return fail(LM_ERR_ARG, "model or src is NULL");
  float* dst = buf_of(m, which);
  if (!dst) return fail(LM_ERR_ARG, "unknown buffer");
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  size_t bytes = (size_t)m->P * 4;
  hipError_t e = hipMemcpyAsync(dst, src, bytes, src_on_device ? hipMemcpyDeviceToDevice : hipMemcpyHostToDevice, s);
  if (e != hipSuccess) return fail(LM_ERR_HIP, std::string("model_set: ") + hipGetErrorString(e));
  {
    // the padding rows of the vocabulary-sized tensors stay zero whatever
    // the caller's gaps hold
    auto zero = [&](long off, long n) {
      if (n > 0) launch_fill_u32(reinterpret_cast<uint32_t*>(dst + off), 0u, n, s);
    };
    zero(m->o_wte + (long)m->V * m->C, (m->Vp - m->V) * m->C);
    if (m->untied) {
      zero(m->o_head_w + (long)m->V * m->C, (m->Vp - m->V) * m->C);
      zero(m->o_head_b + m->V, std::max(m->Vp, m->ldz) - m->V);
    }
  }
  if (which == LM_PARAMS && m->h16) launch_make_shadow(m->params, m->P, m->shadow, m->prec == 2, s);
  if (!src_on_device) {
    e = hipStreamSynchronize(s);
    if (e != hipSuccess) return fail(LM_ERR_HIP, std::string("model_set: ") + hipGetErrorString(e));
  }
  return hip_status("model_set");
}

lm_status model_get(const lm_model* m, lm_buf which, float* dst, int dst_on_device, void* stream) {
  if (!m || !dst) return fail(LM_ERR_ARG, "model or dst is NULL");
  const float* src = buf_of(m, which);
  if (!src) return fail(LM_ERR_ARG, "unknown buffer");
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  hipError_t e = hipMemcpyAsync(dst, src, (size_t)m->P * 4, dst_on_device ? hipMemcpyDeviceToDevice : hipMemcpyDeviceToHost, s);
  if (e == hipSuccess && !dst_on_device) e = hipStreamSynchronize(s);
  if (e != hipSuccess) return fail(LM_ERR_HIP, std::string("model_get: ") + hipGetErrorString(e));
  return LM_OK;
}

lm_status train_step(lm_model* m, const int32_t* tok, const int32_t* tgt, const int32_t* doc, int32_t B, int32_t T,
                     const lm_optim* opt, float* d_stats, void* stream) {
  if (!m || !tok || !tgt || !opt) return fail(LM_ERR_ARG, "model, tokens, targets or optim is NULL");
  lm_status st = check_batch(m, B, T);
  if (st != LM_OK) return st;
  if (opt->step < 1) return fail(LM_ERR_ARG, "optim.step must be >= 1");
  if (!(opt->beta1 >= 0.f && opt->beta1 < 1.f && opt->beta2 >= 0.f && opt->beta2 < 1.f))
    return fail(LM_ERR_ARG, "betas must be in [0, 1)");
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  float* stats = d_stats ? d_stats : m->stats_own;
  Launcher Lr(m, s);
  int rc = 0;
  Lr.run("misc", 0, 0, [&] { launch_fill_u32(m->flags, 0u, 4, s); });
  rc |= with_act(m, [&](auto tag) {
    using E = std::remove_pointer_t<decltype(tag)>;
    return forward_pass<E>(m, Lr, tok, doc, B, T) | backward_pass<E>(m, Lr, tok, tgt, B, T, stats, doc != nullptr);
  });
  if (rc == kTableUploadFailed) return fail(LM_ERR_HIP, "train_step: uploading the weight-gradient table failed");
  if (rc) return fail(LM_ERR_HIP, "internal error: a kernel rejected a shape accepted when the model was created");
  Lr.run("grad_norm", 0, 4.0 * m->P, [&] {
    launch_sumsq_partials(m->grads, m->P, m->norm_part, s);
    launch_norm_finalize(m->norm_part, opt->clip_norm, m->norm_scale, m->flags, stats, m->scaler(), s);
  });
  AdamArgs a{};
  a.p = m->params; a.g = m->grads; a.m = m->adam_m; a.v = m->adam_v; a.n = m->P;
  a.lr = opt->lr; a.beta1 = opt->beta1; a.beta2 = opt->beta2; a.eps = opt->eps; a.wd = opt->weight_decay;
  a.bc1 = (float)(1.0 - std::pow((double)opt->beta1, (double)opt->step));
  a.bc2 = (float)(1.0 - std::pow((double)opt->beta2, (double)opt->step));
  a.norm_scale = m->norm_scale; a.flags = m->flags;
  a.shadow = m->shadow; a.shadow_f16 = m->prec == 2;
  // p, g, m, v read (16 B), p, m, v written (12 B), plus the 16-bit copy (2 B)
  Lr.run("adamw", 0, (m->h16 ? 30.0 : 28.0) * m->P, [&] { launch_adamw(a, s); });
  Lr.run("misc", 0, 0, [&] { launch_write_flags(m->flags, stats, s); });
  return hip_status("train_step");
}

lm_status forward_logits(lm_model* m, const int32_t* tok, const int32_t* doc, int32_t B, int32_t T, float* d_logits,
                         void* stream) {
  if (!m || !tok || !d_logits) return fail(LM_ERR_ARG, "model, tokens or logits is NULL");
  lm_status st = check_batch(m, B, T);
  if (st != LM_OK) return st;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  Launcher Lr(m, s);
  int rc;
  launch_fill_u32(m->flags, 0u, 4, s);
  rc = with_act(m, [&](auto tag) {
    using E = std::remove_pointer_t<decltype(tag)>;
    const int r = forward_pass<E>(m, Lr, tok, doc, B, T);
    launch_logits_out<E>(m->act<E>(m->logits, 0), m->ldz, B * T, m->V, d_logits, s);
    return r;
  });
  if (rc) return fail(LM_ERR_HIP, "internal error: a kernel rejected a shape accepted when the model was created");
  return hip_status("forward_logits");
}

size_t lm_kv_cache_bytes(const lm_config* cfg, int32_t batch) {
  if (!cfg || batch < 1 || lm_workspace_bytes(cfg) == 0) return 0;
  const size_t elem = cfg->precision ? 2 : 4;
  return 2ull * cfg->n_layers * (size_t)batch * cfg->max_seq * cfg->d_model * elem;
}

lm_status model_prefill(lm_model* m, const int32_t* tok, int32_t B, int32_t T, void* d_cache, float* d_logits,
                        void* stream) {
  if (!m || !tok || !d_cache || !d_logits) return fail(LM_ERR_ARG, "model, tokens, cache or logits is NULL");
  lm_status st = check_batch(m, B, T);
  if (st != LM_OK) return st;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  Launcher Lr(m, s);
  const long C = m->C, S = m->S, M = (long)B * T;
  int rc;
  launch_fill_u32(m->flags, 0u, 4, s);
  auto fill = [&](auto* cache) {
    using E = std::remove_pointer_t<decltype(cache)>;
    for (int l = 0; l < m->L; ++l) {
      E* kc = cache + 2L * l * B * S * C;
      launch_kv_store<E>(m->act<E>(m->qkv, l * M * 3 * C), B, T, (int)C, (int)S, 0, kc, kc + (long)B * S * C, s);
    }
    // logits of each row's last position
    launch_logits_out<E>(m->act<E>(m->logits, 0) + (long)(T - 1) * m->ldz, (long)T * m->ldz, B, m->V, d_logits, s);
  };
  rc = with_act(m, [&](auto tag) {
    using E = std::remove_pointer_t<decltype(tag)>;
    const int r = forward_pass<E>(m, Lr, tok, nullptr, B, T);
    fill(reinterpret_cast<E*>(d_cache));
    return r;
  });
  if (rc) return fail(LM_ERR_HIP, "internal error: a kernel rejected a shape accepted when the model was created");
  return hip_status("model_prefill");
}

static lm_status decode_common(lm_model* m, const int32_t* tok, int32_t B, int32_t pos, const int32_t* d_pos,
                               void* d_cache, float* d_logits, void* stream, const char* what) {
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  Launcher Lr(m, s);
  int rc;
  launch_fill_u32(m->flags, 0u, 4, s);
  rc = with_act(m, [&](auto tag) {
    using E = std::remove_pointer_t<decltype(tag)>;
    const int r = decode_pass<E>(m, Lr, tok, B, pos, reinterpret_cast<E*>(d_cache), d_pos);
    launch_logits_out<E>(m->act<E>(m->logits, 0), m->ldz, B, m->V, d_logits, s);
    return r;
  });
  if (rc) return fail(LM_ERR_HIP, "internal error: a kernel rejected a shape accepted when the model was created");
  return hip_status(what);
}

lm_status model_decode(lm_model* m, const int32_t* tok, int32_t B, int32_t pos, void* d_cache, float* d_logits,
                       void* stream) {
  if (!m || !tok || !d_cache || !d_logits) return fail(LM_ERR_ARG, "model, tokens, cache or logits is NULL");
  lm_status st = check_batch(m, B, 1);
  if (st != LM_OK) return st;
  if (pos < 1 || pos >= m->S) return fail(LM_ERR_SHAPE, "pos must be in [1, max_seq): the cache holds positions < pos");
  return decode_common(m, tok, B, pos, nullptr, d_cache, d_logits, stream, "model_decode");
}

lm_status model_decode_at(lm_model* m, const int32_t* tok, int32_t B, const int32_t* d_pos, void* d_cache,
                          float* d_logits, void* stream) {
  if (!m || !tok || !d_pos || !d_cache || !d_logits)
    return fail(LM_ERR_ARG, "model, tokens, position, cache or logits is NULL");
  lm_status st = check_batch(m, B, 1);
  if (st != LM_OK) return st;
  if (m->S < 2) return fail(LM_ERR_SHAPE, "max_seq must be at least 2 to decode");
  return decode_common(m, tok, B, 0, d_pos, d_cache, d_logits, stream, "model_decode_at");
}

lm_status model_set_loss_scaler(lm_model* m, const lm_loss_scaler* ls, void* stream) {
  if (!m || !ls) return fail(LM_ERR_ARG, "model or scaler is NULL");
  if (m->prec != 2) return fail(LM_ERR_UNSUPPORTED, "loss scaling belongs to the fp16 precision (2)");
  if (!(ls->scale > 0.f) || !std::isfinite(ls->scale) || !(ls->growth >= 1.f) || !(ls->backoff > 0.f) ||
      !(ls->backoff <= 1.f) || ls->interval < 1 || ls->good_steps < 0 || ls->good_steps >= ls->interval)
    return fail(LM_ERR_ARG, "loss scaler: need scale > 0 finite, growth >= 1, 0 < backoff <= 1, interval >= 1, "
                            "0 <= good_steps < interval");
  m->ls_growth = ls->growth;
  m->ls_backoff = ls->backoff;
  m->ls_interval = ls->interval;
  const float st[2] = {ls->scale, (float)ls->good_steps};
  hipError_t e = hipMemcpyAsync(m->scale_state, st, sizeof(st), hipMemcpyHostToDevice,
                                reinterpret_cast<hipStream_t>(stream));
  if (e == hipSuccess) e = hipStreamSynchronize(reinterpret_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(LM_ERR_HIP, std::string("model_set_loss_scaler: ") + hipGetErrorString(e));
  return LM_OK;
}

lm_status model_get_loss_scaler(const lm_model* m, lm_loss_scaler* out, void* stream) {
  if (!m || !out) return fail(LM_ERR_ARG, "model or out is NULL");
  if (m->prec != 2) return fail(LM_ERR_UNSUPPORTED, "loss scaling belongs to the fp16 precision (2)");
  float st[2];
  hipError_t e = hipMemcpyAsync(st, m->scale_state, sizeof(st), hipMemcpyDeviceToHost,
                                reinterpret_cast<hipStream_t>(stream));
  if (e == hipSuccess) e = hipStreamSynchronize(reinterpret_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(LM_ERR_HIP, std::string("model_get_loss_scaler: ") + hipGetErrorString(e));
  out->scale = st[0];
  out->good_steps = (int32_t)st[1];
  out->growth = m->ls_growth;
  out->backoff = m->ls_backoff;
  out->interval = m->ls_interval;
  return LM_OK;
}

const char* lm_last_error(void) { return g_err.c_str(); }

lm_status model_profile_enable(lm_model* m, int enable) {
  if (!m) return fail(LM_ERR_ARG, "model is NULL");
  m->prof.drain();
  m->prof.on = enable != 0;
  return LM_OK;
}

lm_status model_profile_read(lm_model* m, lm_profile_entry* out, int32_t cap, int32_t* n, int reset) {
  if (!m || !n) return fail(LM_ERR_ARG, "model or n is NULL");
  m->prof.drain();
  int32_t k = 0;
  for (auto& c : m->prof.cls) {
    if (out && k < cap) {
      std::memset(out[k].name, 0, sizeof(out[k].name));
      std::strncpy(out[k].name, c.name.c_str(), sizeof(out[k].name) - 1);
      out[k].launches = c.launches;
      out[k].ms = c.ms;
      out[k].flops = c.flops;
      out[k].bytes = c.bytes;
    }
    ++k;
  }
  *n = k;
  if (reset)
    for (auto& c : m->prof.cls) c.launches = 0, c.ms = 0, c.flops = 0, c.bytes = 0;
  return LM_OK;
}

}  // extern "C"
