// C-ABI entry points of libec.so: argument checks (ec_validate.cpp), workspace
// sizes and carving, and kernel launches on the caller's stream.  No entry
// point allocates device memory, synchronises, or reads device memory on the
// host.
#include "ec.h"

#include <math.h>
#include <string.h>

#include "ec_launch.h"
#include "ec_validate.h"

namespace {

using ec::dtype_ok;
inline bool al16(const void* p) { return ec::aligned16(p); }
inline size_t up256(size_t b) { return (b + 255) & ~size_t(255); }
inline size_t esize(int32_t dtype) { return ec::elem_size(dtype); }
inline int32_t launch_status(hipError_t e) {
  if (e == hipSuccess) return EC_OK;
  if (e == hipErrorNotSupported) return EC_E_UNSUPPORTED;
  return EC_E_LAUNCH;
}
#define EC_TRY(expr)                                 \
  do {                                               \
    const int32_t _st = launch_status(expr);         \
    if (_st != EC_OK) return _st;                    \
  } while (0)

// Bump allocator over the caller's workspace.
struct Carver {
  char* base;
  size_t off = 0;
  explicit Carver(void* p) : base(static_cast<char*>(p)) {}
  template <typename T> T* take(size_t bytes) {
    T* p = reinterpret_cast<T*>(base ? base + off : nullptr);
    off += up256(bytes);
    return p;
  }
};

}  // namespace

namespace {
ec::GemmArgs qkv_args(int32_t max_rows, int32_t d, int32_t Hq, int32_t Hkv, int32_t dh,
                      int32_t dtype) {
  ec::GemmArgs g;
  g.dtype = dtype; g.epi = ec::Epi::kQKV; g.max_rows = max_rows; g.N = (Hq + 2 * Hkv) * dh;
  g.K = d; g.Hq = Hq; g.Hkv = Hkv; g.dh = dh;
  return g;
}
}  // namespace

extern "C" {

const char* ec_status_string(int32_t s) {
  switch (s) {
    case EC_OK: return "ok";
    case EC_E_NULL: return "a required pointer is NULL";
    case EC_E_SHAPE: return "a size is out of range or inconsistent";
    case EC_E_DTYPE: return "unknown dtype";
    case EC_E_WORKSPACE: return "workspace too small";
    case EC_E_ALIGN: return "pointer or stride not 16-byte aligned";
    case EC_E_LAUNCH: return "kernel launch failed";
    case EC_E_UNSUPPORTED: return "unsupported size or combination";
    default: return "unknown status";
  }
}

int32_t ec_abi_version(void) { return EC_ABI_VERSION; }

// ---------------------------------------------------------------- entropy pass
size_t ec_entropy_workspace_bytes(int64_t n_rows, int64_t V) {
  if (n_rows < 1 || V < 1) return 0;
  // sized for the finer (fp32) segmentation, so one workspace serves both dtypes
  return up256(ec::entropy_ws_bytes(n_rows, V, EC_F32));
}

int32_t ec_entropy_max(const void* logits, int32_t dtype, int64_t n_rows, int64_t V,
                       int64_t row_stride, const int32_t* decoded_rows, const int32_t* n_decoded,
                       int32_t max_decoded, float tau, float* row_entropy, int32_t* row_argmax,
                       float* row_top1, float* e_max, int32_t* full_flag, void* ws,
                       size_t ws_bytes, hipStream_t stream) {
  if (!ws) return EC_E_NULL;
  const int32_t st = ec::check_entropy(logits, dtype, n_rows, V, row_stride, decoded_rows,
                                       n_decoded, max_decoded, row_entropy, e_max, full_flag);
  if (st != EC_OK) return st;
  if (!al16(ws)) return EC_E_ALIGN;
  if (ws_bytes < ec_entropy_workspace_bytes(n_rows, V)) return EC_E_WORKSPACE;
  EC_TRY(ec::launch_entropy(logits, dtype, n_rows, nullptr, V, row_stride, row_entropy,
                            row_argmax, row_top1, decoded_rows, n_decoded, max_decoded, tau, e_max,
                            full_flag, ws, stream));
  return EC_OK;
}

// ------------------------------------------------------------------ selection
int32_t ec_select_rows(const int32_t* full_flag, const uint8_t* is_masked, int32_t L,
                       int32_t block_start, int32_t block_len, int32_t block_causal,
                       const int32_t* history, const int32_t* history_len, int32_t history_cap,
                       int32_t k, int32_t* rows, int32_t* n_rows, hipStream_t stream) {
  const int32_t st = ec::check_select(full_flag, is_masked, L, block_start, block_len,
                                      block_causal, history, history_len, history_cap, k, rows,
                                      n_rows);
  if (st != EC_OK) return st;
  EC_TRY(ec::launch_select_rows(full_flag, is_masked, L, block_start, block_len, block_causal,
                                history, history_len, history_cap, k, rows, n_rows, nullptr,
                                nullptr, nullptr, stream));
  return EC_OK;
}

// ------------------------------------------------------------------ KV refresh

size_t ec_kv_refresh_workspace_bytes(int32_t max_rows, int32_t d, int32_t Hq, int32_t Hkv,
                                     int32_t dh, int32_t dtype) {
  if (max_rows < 1 || d < 1 || Hq < 1 || Hkv < 1 || dh < 1 || !dtype_ok(dtype)) return 0;
  return ec::gemm_ws_bytes(qkv_args(max_rows, d, Hq, Hkv, dh, dtype));
}

int32_t ec_kv_refresh(const void* x, int64_t x_stride, const int32_t* rows, const int32_t* n_rows,
                      int32_t max_rows, const void* w_qkv, int32_t d, int32_t Hq, int32_t Hkv,
                      int32_t dh, int32_t dtype, void* q_out, void* k_cache, void* v_cache,
                      int32_t L_cap, void* ws, size_t ws_bytes, hipStream_t stream) {
  const int32_t st = ec::check_refresh(x, x_stride, rows, n_rows, max_rows, w_qkv, d, Hq, Hkv, dh,
                                       dtype, q_out, k_cache, v_cache, L_cap, ws);
  if (st != EC_OK) return st;
  ec::GemmArgs g = qkv_args(max_rows, d, Hq, Hkv, dh, dtype);
  const size_t need = ec::gemm_ws_bytes(g);
  if (need > 0 && !ws) return EC_E_NULL;
  if (ws_bytes < need) return EC_E_WORKSPACE;
  g.A = x; g.lda = x_stride; g.n_rows_dev = n_rows; g.W = w_qkv; g.rows = rows; g.q_out = q_out;
  g.k_cache = k_cache; g.v_cache = v_cache; g.L_cap = L_cap;
  EC_TRY(ec::launch_gemm_rows(g, ws, stream));
  return EC_OK;
}

// ------------------------------------------------------------------ attention
size_t ec_attention_workspace_bytes(int32_t max_rows, int32_t L, int32_t Hq, int32_t Hkv,
                                    int32_t dh) {
  if (max_rows < 1 || L < 1 || Hq < 1 || Hkv < 1 || dh < 1) return 0;
  return up256(ec::attn_ws_bytes(max_rows, L, Hq, Hkv, dh));
}

int32_t ec_bidir_attention(const void* q, const int32_t* n_rows, int32_t max_rows,
                           const void* k_cache, const void* v_cache, int32_t L, int32_t L_cap,
                           int32_t Hq, int32_t Hkv, int32_t dh, float scale, int32_t dtype,
                           void* out, void* ws, size_t ws_bytes, hipStream_t stream) {
  const int32_t st = ec::check_attention(q, n_rows, max_rows, k_cache, v_cache, L, L_cap, Hq, Hkv,
                                         dh, scale, dtype, out, ws);
  if (st != EC_OK) return st;
  const size_t need = ec_attention_workspace_bytes(max_rows, L, Hq, Hkv, dh);
  if (need > 0 && !ws) return EC_E_NULL;
  if (ws_bytes < need) return EC_E_WORKSPACE;
  ec::AttnArgs a;
  a.dtype = dtype; a.q = q; a.n_rows_dev = n_rows; a.max_rows = max_rows; a.k_cache = k_cache;
  a.v_cache = v_cache; a.L = L; a.L_cap = L_cap; a.Hq = Hq; a.Hkv = Hkv; a.dh = dh;
  a.scale = scale; a.out = out;
  EC_TRY(ec::launch_attention(a, ws, stream));
  return EC_OK;
}

}  // extern "C"

// ------------------------------------------------------------------ full step
namespace {

struct StepLayout {
  size_t total = 0;
  void* x = nullptr;        // [L_cap, d]        activations of the selected rows
  void* a = nullptr;        // [L_cap, d]        normed activations (d_ffn > 0)
  void* q = nullptr;        // [L_cap, Hq*dh]
  void* o = nullptr;        // [L_cap, Hq*dh]    attention output
  void* h = nullptr;        // [L_cap, d_ffn]    FFN intermediate (d_ffn > 0)
  void* attn_ws = nullptr;
  void* gemm_ws = nullptr;
  void* ent_ws = nullptr;
  void* drift_ws = nullptr;   // stale Value cache of one layer + per-position distances
  int32_t* cand_pos = nullptr;
  int32_t* cand_idx = nullptr;
  int32_t* n_cand = nullptr;
};

StepLayout step_layout(const ec_model* m, int32_t max_block, void* ws) {
  const size_t es = esize(m->dtype);
  const size_t L = size_t(m->L_cap), d = size_t(m->d), hd = size_t(m->Hq) * m->dh;
  Carver c(ws);
  StepLayout s;
  s.x = c.take<void>(L * d * es);
  if (m->d_ffn) s.a = c.take<void>(L * d * es);
  s.q = c.take<void>(L * hd * es);
  s.o = c.take<void>(L * hd * es);
  if (m->d_ffn) s.h = c.take<void>(L * size_t(m->d_ffn) * es);
  s.attn_ws = c.take<void>(ec::attn_ws_bytes(m->L_cap, m->L_cap, m->Hq, m->Hkv, m->dh));
  // one split-K buffer serves every GEMM of the step (they run one after another)
  size_t gws = 0;
  auto need = [&](ec::Epi epi, int rows, int N, int K) {
    ec::GemmArgs g;
    g.dtype = m->dtype; g.epi = epi; g.max_rows = rows; g.N = N; g.K = K;
    const size_t b = ec::gemm_ws_bytes(g);
    if (b > gws) gws = b;
  };
  need(ec::Epi::kQKV, m->L_cap, (m->Hq + 2 * m->Hkv) * m->dh, m->d);
  need(ec::Epi::kResidual, m->L_cap, m->d, m->Hq * m->dh);
  if (m->d_ffn) {
    need(ec::Epi::kSwiGLU, m->L_cap, m->d_ffn, m->d);
    need(ec::Epi::kResidual, m->L_cap, m->d, m->d_ffn);
  }
  if (m->w_lm) need(ec::Epi::kLogits, max_block, m->V, m->d);
  s.gemm_ws = c.take<void>(gws);
  // entropy partials: the entropy pass's segments, or the packed LM head's
  // per-(row, tile group) statistics (one region serves both).  The latter
  // is sized for min(max_block, kLmStatRows) rows whatever max_block, so a
  // workspace sized for a larger bound also serves blocks of at most
  // kLmStatRows positions without a logits buffer.
  size_t ent = ec::entropy_ws_bytes(max_block, m->V, m->dtype);
  if (m->w_lm && m->w_lm_packed) {
    const size_t rows = size_t(max_block < ec::kLmStatRows ? max_block : ec::kLmStatRows);
    const size_t lm = rows * size_t(ec::lmhead_max_stat_groups(m->V)) * sizeof(ec::EntropyPartial);
    if (lm > ent) ent = lm;
  }
  s.ent_ws = c.take<void>(ent);
  s.drift_ws = c.take<void>(ec::value_drift_ws_bytes(m->dtype, m->Hkv * m->dh, m->L_cap));
  s.cand_pos = c.take<int32_t>(size_t(max_block) * 4);
  s.cand_idx = c.take<int32_t>(size_t(max_block) * 4);
  s.n_cand = c.take<int32_t>(4);
  s.total = c.off;
  return s;
}

struct PhaseTimer {
  hipEvent_t* ev;
  hipStream_t s;
  hipError_t begin(int p) const { return (ev && ev[2 * p]) ? hipEventRecord(ev[2 * p], s) : hipSuccess; }
  hipError_t end(int p) const { return (ev && ev[2 * p + 1]) ? hipEventRecord(ev[2 * p + 1], s) : hipSuccess; }
};

}  // namespace

extern "C" {

int32_t ec_pack_lm_head(const void* w_lm, int32_t V, int32_t d, int32_t dtype, void* w_packed,
                        hipStream_t stream) {
  const int32_t st = ec::check_pack(w_lm, V, d, dtype, w_packed);
  if (st != EC_OK) return st;
  EC_TRY(ec::launch_pack_fragments(w_lm, V, d, w_packed, stream));
  return EC_OK;
}

size_t ec_step_workspace_bytes(const ec_model* m, int32_t max_block) {
  if (!m || !ec::model_ok(m) || !dtype_ok(m->dtype) || max_block < 1) return 0;
  return step_layout(m, max_block, nullptr).total;
}

int32_t ec_step(const ec_model* m, const ec_state* st, const ec_step_cfg* c, void* ws,
                size_t ws_bytes, hipEvent_t* phase_events, hipStream_t stream) {
  const int32_t chk = ec::check_step(m, st, c, ws);
  if (chk != EC_OK) return chk;
  const bool external = (m->w_lm == nullptr);   // no LM head: the caller decodes
  const int32_t max_block = c->block_len;
  const StepLayout s = step_layout(m, max_block, ws);
  if (ws_bytes < s.total) return EC_E_WORKSPACE;

  const int dt = m->dtype;
  const int L = st->L;
  const int hd = m->Hq * m->dh;
  // A full step selects all L rows (block diffusion: the block_len rows of
  // the current block); a partial step at most block_len + k (the block's
  // masked positions and the last k decoded ones; block diffusion: those in
  // the block).  The small-row kernels see a full step only when it selects
  // at most kSmallMaxRows rows.
  const bool causal = c->block_causal != 0;
  const int full_rows = causal ? c->block_len : L;
  const int64_t part_rows = causal ? int64_t(c->block_len) : int64_t(c->block_len) + c->k;
  const int part_hi = part_rows >= full_rows ? full_rows : int(part_rows);
  const int sk_rows = full_rows <= ec::kSmallMaxRows ? full_rows : part_hi;
  // The most rows this step can select, and the row-count paths it can reach
  // (a caller-stated mode leaves out the other mode's kernels).
  const int hi = c->mode == EC_MODE_PARTIAL ? part_hi : full_rows;
  unsigned paths = 0;
  if (c->mode != EC_MODE_FULL || full_rows <= ec::kSmallMaxRows) paths |= ec::kPathSmall;
  if (hi > ec::kSmallMaxRows) paths |= ec::kPathLarge;
  // Keys each recomputed row attends to: the whole sequence, or (block
  // diffusion) the positions before the current block's end.
  const int L_keys = causal ? c->block_start + c->block_len : L;
  const bool maybe_full = c->mode != EC_MODE_PARTIAL;
  const PhaseTimer tm{phase_events, stream};

  EC_TRY(tm.begin(EC_PHASE_SELECT));
  EC_TRY(ec::launch_select_rows(st->full_flag, st->is_masked, L, c->block_start, c->block_len,
                                c->block_causal, st->history, st->history_len, st->history_cap,
                                c->k, st->rows, st->n_rows, s.cand_pos, s.cand_idx, s.n_cand,
                                stream));
  EC_TRY(tm.end(EC_PHASE_SELECT));
  EC_TRY(tm.begin(EC_PHASE_EMBED));
  EC_TRY(ec::launch_embed(dt, m->tok_emb, m->pos_emb, st->tokens, st->rows, st->n_rows, hi, m->d,
                          s.x, stream));
  EC_TRY(tm.end(EC_PHASE_EMBED));

  for (int l = 0; l < m->n_layers; ++l) {
    const ec_layer& ly = m->layers[l];
    const bool first = (l == 0);
    const void* a_in = s.x;
    if (first) EC_TRY(tm.begin(EC_PHASE_QKV));
    if (m->d_ffn) {
      EC_TRY(ec::launch_rmsnorm(dt, s.x, st->n_rows, hi, m->d, ly.norm_attn, m->rms_eps, s.a, stream));
      a_in = s.a;
    }
    ec::GemmArgs g;
    g.dtype = dt; g.epi = ec::Epi::kQKV; g.A = a_in; g.lda = m->d; g.n_rows_dev = st->n_rows;
    g.max_rows = hi; g.skinny_rows = sk_rows; g.paths = paths; g.W = ly.w_qkv; g.N = (m->Hq + 2 * m->Hkv) * m->dh; g.K = m->d;
    g.rows = st->rows; g.q_out = s.q; g.k_cache = st->k_cache[l]; g.v_cache = st->v_cache[l];
    g.Hq = m->Hq; g.Hkv = m->Hkv; g.dh = m->dh; g.L_cap = m->L_cap;
    const int vrows = m->Hkv * m->dh;
    if (st->kv_drift && maybe_full)   // full steps only (the kernels read the flag): the stale Value cache
      EC_TRY(ec::launch_value_drift_snapshot(dt, st->full_flag, st->v_cache[l], vrows, L, m->L_cap,
                                             s.drift_ws, stream));
    EC_TRY(ec::launch_gemm_rows(g, s.gemm_ws, stream));
    if (st->kv_drift && maybe_full)
      EC_TRY(ec::launch_value_drift(dt, st->full_flag, st->v_cache[l], vrows, L, m->L_cap, s.drift_ws,
                                    st->kv_drift + 2 * l, stream));
    if (first) { EC_TRY(tm.end(EC_PHASE_QKV)); EC_TRY(tm.begin(EC_PHASE_ATTN)); }

    ec::AttnArgs a;
    a.dtype = dt; a.q = s.q; a.n_rows_dev = st->n_rows; a.max_rows = hi; a.k_cache = st->k_cache[l];
    a.v_cache = st->v_cache[l]; a.L = L_keys; a.L_cap = m->L_cap; a.Hq = m->Hq; a.Hkv = m->Hkv;
    a.dh = m->dh; a.scale = 1.0f / sqrtf(float(m->dh)); a.out = s.o; a.paths = paths;
    a.small_rows = sk_rows;
    EC_TRY(ec::launch_attention(a, s.attn_ws, stream));
    if (first) { EC_TRY(tm.end(EC_PHASE_ATTN)); EC_TRY(tm.begin(EC_PHASE_OPROJ)); }

    ec::GemmArgs go;
    go.dtype = dt; go.epi = ec::Epi::kResidual; go.A = s.o; go.lda = hd; go.n_rows_dev = st->n_rows;
    go.max_rows = hi; go.skinny_rows = sk_rows; go.paths = paths; go.W = ly.w_o; go.N = m->d; go.K = hd; go.C = s.x; go.ldc = m->d;
    EC_TRY(ec::launch_gemm_rows(go, s.gemm_ws, stream));
    if (first) EC_TRY(tm.end(EC_PHASE_OPROJ));

    if (m->d_ffn) {
      if (first) EC_TRY(tm.begin(EC_PHASE_FFN));
      EC_TRY(ec::launch_rmsnorm(dt, s.x, st->n_rows, hi, m->d, ly.norm_ffn, m->rms_eps, s.a, stream));
      ec::GemmArgs gu;
      gu.dtype = dt; gu.epi = ec::Epi::kSwiGLU; gu.A = s.a; gu.lda = m->d;
      gu.n_rows_dev = st->n_rows; gu.max_rows = hi; gu.skinny_rows = sk_rows; gu.paths = paths; gu.W = ly.w_gate; gu.W2 = ly.w_up;
      gu.N = m->d_ffn; gu.K = m->d; gu.C = s.h; gu.ldc = m->d_ffn;
      EC_TRY(ec::launch_gemm_rows(gu, s.gemm_ws, stream));
      ec::GemmArgs gd;
      gd.dtype = dt; gd.epi = ec::Epi::kResidual; gd.A = s.h; gd.lda = m->d_ffn;
      gd.n_rows_dev = st->n_rows; gd.max_rows = hi; gd.skinny_rows = sk_rows; gd.paths = paths; gd.W = ly.w_down; gd.N = m->d; gd.K = m->d_ffn;
      gd.C = s.x; gd.ldc = m->d;
      EC_TRY(ec::launch_gemm_rows(gd, s.gemm_ws, stream));
      if (first) EC_TRY(tm.end(EC_PHASE_FFN));
    }
  }

  if (st->attn_out)   // rows past *n_rows carry whatever the workspace held
    EC_TRY(hipMemcpyAsync(st->attn_out, s.o, size_t(hi) * size_t(hd) * esize(dt),
                          hipMemcpyDeviceToDevice, stream));

  if (external) {
    // The caller decoded c->n_unmask rows itself and left their logits in
    // st->logits: take E over all of them and decide; tokens, mask and
    // history stay as they are.
    EC_TRY(tm.begin(EC_PHASE_LMHEAD));
    EC_TRY(tm.end(EC_PHASE_LMHEAD));
    // One timed phase covers the entropy pass and the decision (one kernel).
    EC_TRY(tm.begin(EC_PHASE_ENTROPY));
    EC_TRY(ec::launch_entropy_step(st->logits, dt, c->n_unmask, nullptr, m->V, m->V,
                                   st->row_entropy, st->row_argmax, st->row_top1, nullptr, 0,
                                   c->tau, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, 0,
                                   st->e_max, st->full_flag, s.ent_ws, stream));
    EC_TRY(tm.end(EC_PHASE_ENTROPY));
    EC_TRY(tm.begin(EC_PHASE_DECIDE));
    EC_TRY(tm.end(EC_PHASE_DECIDE));
    return EC_OK;
  }

  EC_TRY(tm.begin(EC_PHASE_LMHEAD));
  const void* xf = s.x;
  if (m->d_ffn) {
    EC_TRY(ec::launch_rmsnorm(dt, s.x, st->n_rows, hi, m->d, m->norm_final, m->rms_eps, s.a, stream));
    xf = s.a;
  }
  ec::GemmArgs gl;
  gl.dtype = dt; gl.epi = ec::Epi::kLogits; gl.A = xf; gl.lda = m->d; gl.a_idx = s.cand_idx;
  gl.n_rows_dev = s.n_cand; gl.max_rows = max_block; gl.W = m->w_lm; gl.N = m->V; gl.K = m->d;
  gl.C = st->logits; gl.ldc = m->V; gl.scale = m->logit_scale; gl.scale_pos = s.cand_pos;
  gl.W_packed = m->w_lm_packed;
  // Without a logits buffer the packed LM head writes each row's softmax
  // statistics instead of its logits (the argument checks admit that only
  // where the packed kernel runs)
  int stat_groups = 0;
  if (st->logits == nullptr) {
    gl.stats = static_cast<ec::EntropyPartial*>(s.ent_ws);
    gl.stats_groups = &stat_groups;
  }
  EC_TRY(ec::launch_gemm_rows(gl, s.gemm_ws, stream));
  EC_TRY(tm.end(EC_PHASE_LMHEAD));
  if (st->logits == nullptr && stat_groups == 0) return EC_E_LAUNCH;   // not reached after the checks

  // The entropy phase now includes the unmask choice and the decision, which
  // run in the same kernel as the per-row fold (the decide phase is empty).
  // From the LM head's statistics, or the entropy pass over the logits.
  EC_TRY(tm.begin(EC_PHASE_ENTROPY));
  if (stat_groups > 0)
    EC_TRY(ec::launch_entropy_step_fused(static_cast<const ec::EntropyPartial*>(s.ent_ws), stat_groups,
                                         max_block, s.n_cand, st->row_entropy, st->row_argmax,
                                         st->row_top1, s.cand_pos, c->n_unmask, c->tau, st->chosen,
                                         st->n_chosen, st->tokens, st->is_masked, st->history,
                                         st->history_len, st->history_cap, st->e_max, st->full_flag,
                                         stream));
  else
    EC_TRY(ec::launch_entropy_step(st->logits, dt, max_block, s.n_cand, m->V, m->V,
                                   st->row_entropy, st->row_argmax, st->row_top1, s.cand_pos,
                                   c->n_unmask, c->tau, st->chosen, st->n_chosen, st->tokens,
                                   st->is_masked, st->history, st->history_len, st->history_cap,
                                   st->e_max, st->full_flag, s.ent_ws, stream));
  EC_TRY(tm.end(EC_PHASE_ENTROPY));
  EC_TRY(tm.begin(EC_PHASE_DECIDE));
  EC_TRY(tm.end(EC_PHASE_DECIDE));
  return EC_OK;
}

}  // extern "C"
