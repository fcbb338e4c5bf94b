// Host-side argument checks of the C ABI (see ec_validate.h).  No HIP call or
// device code here: this file also builds with a plain host compiler and the
// address / undefined-behaviour sanitizers.
#include "ec_validate.h"

#include <math.h>
#include <stdint.h>

#include "ec_limits.h"

namespace ec {

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
size_t elem_size(int32_t dtype) { return dtype == EC_BF16 ? 2 : 4; }
bool dtype_ok(int32_t dtype) { return dtype == EC_F32 || dtype == EC_BF16; }

int32_t check_entropy(const void* logits, int32_t dtype, int64_t n_rows, int64_t V,
                      int64_t row_stride, const int32_t* decoded_rows, const int32_t* n_decoded,
                      int32_t max_decoded, const float* row_entropy, const float* e_max,
                      const int32_t* full_flag) {
  if (!logits || !row_entropy || !e_max || !full_flag) return EC_E_NULL;
  if (decoded_rows && !n_decoded) return EC_E_NULL;
  if (!dtype_ok(dtype)) return EC_E_DTYPE;
  if (n_rows < 1 || V < 1 || row_stride < V || max_decoded < 0) return EC_E_SHAPE;
  if (n_rows > (int64_t(1) << 24) || V > (int64_t(1) << 30) || row_stride > (int64_t(1) << 40))
    return EC_E_UNSUPPORTED;
  if (!aligned16(logits) || (row_stride * int64_t(elem_size(dtype))) % 16 != 0) return EC_E_ALIGN;
  return EC_OK;
}

int32_t check_select(const int32_t* full_flag, const uint8_t* is_masked, int32_t L,
                     int32_t block_start, int32_t block_len, int32_t block_causal,
                     const int32_t* history, const int32_t* history_len, int32_t history_cap,
                     int32_t k, const int32_t* rows, const int32_t* n_rows) {
  if (!full_flag || !is_masked || !history || !history_len || !rows || !n_rows) return EC_E_NULL;
  if (L < 1 || block_start < -1 || block_len < 0 || block_len > L ||
      (block_start >= 0 && int64_t(block_start) + block_len > L) || k < 0 || history_cap < 1 ||
      k > history_cap || (block_causal != 0 && block_causal != 1) ||
      (block_causal && block_start < 0))
    return EC_E_SHAPE;
  if (L > kSelectMaxL) return EC_E_UNSUPPORTED;
  return EC_OK;
}

int32_t check_refresh(const void* x, int64_t x_stride, const int32_t* rows, const int32_t* n_rows,
                      int32_t max_rows, const void* w_qkv, int32_t d, int32_t Hq, int32_t Hkv,
                      int32_t dh, int32_t dtype, const void* q_out, const void* k_cache,
                      const void* v_cache, int32_t L_cap, const void* ws) {
  if (!x || !rows || !n_rows || !w_qkv || !q_out || !k_cache || !v_cache) return EC_E_NULL;
  if (!dtype_ok(dtype)) return EC_E_DTYPE;
  if (max_rows < 1 || d < 1 || Hq < 1 || Hkv < 1 || dh < 1 || L_cap < 1 || x_stride < d ||
      Hq % Hkv != 0)
    return EC_E_SHAPE;
  if (d % k_multiple(dtype) != 0 || !head_dim_ok(dh) || x_stride > (int64_t(1) << 40) ||
      int64_t(Hq + 2 * int64_t(Hkv)) * dh > (int64_t(1) << 30))
    return EC_E_UNSUPPORTED;
  if (!aligned16(x) || !aligned16(w_qkv) || !aligned16(q_out) || !aligned16(k_cache) ||
      !aligned16(v_cache) || (ws && !aligned16(ws)) ||
      (x_stride * int64_t(elem_size(dtype))) % 16 != 0)
    return EC_E_ALIGN;
  return EC_OK;
}

int32_t check_attention(const void* q, const int32_t* n_rows, int32_t max_rows,
                        const void* k_cache, const void* v_cache, int32_t L, int32_t L_cap,
                        int32_t Hq, int32_t Hkv, int32_t dh, float scale, int32_t dtype,
                        const void* out, const void* ws) {
  if (!q || !n_rows || !k_cache || !v_cache || !out) return EC_E_NULL;
  if (!dtype_ok(dtype)) return EC_E_DTYPE;
  if (max_rows < 1 || L < 1 || L > L_cap || Hq < 1 || Hkv < 1 || dh < 1 || Hq % Hkv != 0 ||
      !(scale > 0.f) || !isfinite(scale))
    return EC_E_SHAPE;
  if (!head_dim_ok(dh) || Hq / Hkv > kMaxGroup) return EC_E_UNSUPPORTED;
  if (!aligned16(q) || !aligned16(k_cache) || !aligned16(v_cache) || !aligned16(out) ||
      (ws && !aligned16(ws)) || (int64_t(L_cap) * int64_t(elem_size(dtype))) % 16 != 0)
    return EC_E_ALIGN;
  return EC_OK;
}

bool model_ok(const ec_model* m) {
  return m->n_layers >= 1 && m->d >= 64 && m->Hq >= 1 && m->Hkv >= 1 && m->dh >= 1 &&
         m->Hq % m->Hkv == 0 && m->V >= 1 && m->L_cap >= 1 && m->d_ffn >= 0;
}

int32_t check_pack(const void* w_lm, int32_t V, int32_t d, int32_t dtype, const void* w_packed) {
  if (!w_lm || !w_packed) return EC_E_NULL;
  if (dtype != EC_BF16) return EC_E_DTYPE;
  if (V < 16 || V % 16 != 0 || d < 32 || d % 32 != 0) return EC_E_SHAPE;
  if (int64_t(V) * d > (int64_t(1) << 40)) return EC_E_UNSUPPORTED;
  if (!aligned16(w_lm) || !aligned16(w_packed)) return EC_E_ALIGN;
  const uintptr_t a = reinterpret_cast<uintptr_t>(w_lm), b = reinterpret_cast<uintptr_t>(w_packed);
  const uintptr_t n = uintptr_t(int64_t(V) * d * 2);
  if (a < b + n && b < a + n) return EC_E_SHAPE;              // the copy may not overlap its source
  return EC_OK;
}

int32_t check_step(const ec_model* m, const ec_state* st, const ec_step_cfg* c, const void* ws) {
  if (!m || !st || !c || !ws) return EC_E_NULL;
  if (!dtype_ok(m->dtype)) return EC_E_DTYPE;
  if (!model_ok(m)) return EC_E_SHAPE;
  if (!m->tok_emb || !m->pos_emb || !m->layers) return EC_E_NULL;
  const bool external = (m->w_lm == nullptr);   // no LM head: the caller decodes
  if (m->d_ffn && !external && !m->norm_final) return EC_E_NULL;
  for (int l = 0; l < m->n_layers; ++l) {
    const ec_layer& ly = m->layers[l];
    if (!ly.w_qkv || !ly.w_o) return EC_E_NULL;
    if (m->d_ffn && (!ly.norm_attn || !ly.norm_ffn || !ly.w_gate || !ly.w_up || !ly.w_down))
      return EC_E_NULL;
  }
  // Without a logits buffer the step folds the softmax statistics that the
  // packed LM head writes in place of its logits: a model without LM head
  // (whose caller supplies logits) or without the packed copy needs one.
  const bool no_logits = (st->logits == nullptr);
  if (no_logits && (external || !m->w_lm_packed)) return EC_E_NULL;
  if (!st->tokens || !st->is_masked || !st->history || !st->history_len || !st->full_flag ||
      !st->k_cache || !st->v_cache || !st->rows || !st->n_rows ||
      !st->row_entropy || !st->row_argmax || !st->row_top1 || !st->chosen || !st->n_chosen ||
      !st->e_max)
    return EC_E_NULL;
  for (int l = 0; l < m->n_layers; ++l)
    if (!st->k_cache[l] || !st->v_cache[l]) return EC_E_NULL;
  if (st->L < 1 || st->L > m->L_cap || c->block_start < -1 || c->block_len < 1 ||
      c->block_len > st->L ||
      (c->block_start >= 0 && int64_t(c->block_start) + c->block_len > st->L) || c->k < 0 ||
      c->k > st->history_cap || c->n_unmask < 0 || st->history_cap < 1 ||
      (c->mode != EC_MODE_DEVICE && c->mode != EC_MODE_FULL && c->mode != EC_MODE_PARTIAL) ||
      (c->block_causal != 0 && c->block_causal != 1) || (c->block_causal && c->block_start < 0))
    return EC_E_SHAPE;
  if (external && (c->n_unmask < 1 || c->n_unmask > c->block_len)) return EC_E_SHAPE;
  const int km = k_multiple(m->dtype);
  if (m->d % km != 0 || (int64_t(m->Hq) * m->dh) % km != 0 || m->d_ffn % km != 0 ||
      m->d_ffn % 32 != 0 || !head_dim_ok(m->dh) || m->Hq / m->Hkv > kMaxGroup ||
      c->block_len > kStepMaxRows || st->L > kSelectMaxL || m->L_cap > kSelectMaxL ||
      m->n_layers > 4096 || int64_t(m->Hq) * m->dh > (int64_t(1) << 20) ||
      m->V > (1 << 30) || (!external && m->V % 32 != 0) ||   // the LM head's GEMM takes whole 32-column blocks
      (no_logits && (c->block_len > kLmStatRows || (int64_t(m->V) + 63) / 64 < kLmMinTiles ||
                     m->d % kLmKBlock != 0)))                // where the packed kernel does not run
    return EC_E_UNSUPPORTED;
  if (!aligned16(ws) || !aligned16(m->tok_emb) || !aligned16(m->pos_emb) ||
      (!external && !aligned16(m->w_lm)) || (!no_logits && !aligned16(st->logits)) ||
      (int64_t(m->V) * int64_t(elem_size(m->dtype))) % 16 != 0 ||
      (int64_t(m->L_cap) * int64_t(elem_size(m->dtype))) % 16 != 0)
    return EC_E_ALIGN;
  if (m->d_ffn && !external && !aligned16(m->norm_final)) return EC_E_ALIGN;
  if (m->w_lm_packed) {
    if (external) return EC_E_NULL;                          // a packed copy of no LM head
    if (m->dtype != EC_BF16) return EC_E_DTYPE;
    if (m->V % 16 != 0) return EC_E_SHAPE;
    if (!aligned16(m->w_lm_packed)) return EC_E_ALIGN;
  }
  if (st->attn_out && !aligned16(st->attn_out)) return EC_E_ALIGN;
  for (int l = 0; l < m->n_layers; ++l) {
    const ec_layer& ly = m->layers[l];
    if (!aligned16(st->k_cache[l]) || !aligned16(st->v_cache[l]) || !aligned16(ly.w_qkv) ||
        !aligned16(ly.w_o))
      return EC_E_ALIGN;
    if (m->d_ffn && (!aligned16(ly.norm_attn) || !aligned16(ly.norm_ffn) ||
                     !aligned16(ly.w_gate) || !aligned16(ly.w_up) || !aligned16(ly.w_down)))
      return EC_E_ALIGN;
  }
  return EC_OK;
}

}  // namespace ec
