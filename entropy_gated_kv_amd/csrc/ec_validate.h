// Host-side argument checks of the C ABI, in a translation unit of their own
// that builds without HIP device code or runtime calls (only the declarations
// of ec.h), so that a host compiler with address and undefined-behaviour
// sanitizers can build and exercise them.  Each returns EC_OK or the status
// the entry point reports; workspace sizes, which depend on kernel plans, are
// checked by the entry points themselves.
#pragma once
#include "ec.h"

namespace ec {

bool aligned16(const void* p);
size_t elem_size(int32_t dtype);
bool dtype_ok(int32_t dtype);

int32_t check_entropy(const void* logits, int32_t dtype, int64_t n_rows, int64_t V,
                      int64_t row_stride, const int32_t* decoded_rows, const int32_t* n_decoded,
                      int32_t max_decoded, const float* row_entropy, const float* e_max,
                      const int32_t* full_flag);
// ec_pack_lm_head
int32_t check_pack(const void* w_lm, int32_t V, int32_t d, int32_t dtype, const void* w_packed);
int32_t check_select(const int32_t* full_flag, const uint8_t* is_masked, int32_t L,
                     int32_t block_start, int32_t block_len, int32_t block_causal,
                     const int32_t* history, const int32_t* history_len, int32_t history_cap,
                     int32_t k, const int32_t* rows, const int32_t* n_rows);
int32_t check_refresh(const void* x, int64_t x_stride, const int32_t* rows, const int32_t* n_rows,
                      int32_t max_rows, const void* w_qkv, int32_t d, int32_t Hq, int32_t Hkv,
                      int32_t dh, int32_t dtype, const void* q_out, const void* k_cache,
                      const void* v_cache, int32_t L_cap, const void* ws);
int32_t check_attention(const void* q, const int32_t* n_rows, int32_t max_rows,
                        const void* k_cache, const void* v_cache, int32_t L, int32_t L_cap,
                        int32_t Hq, int32_t Hkv, int32_t dh, float scale, int32_t dtype,
                        const void* out, const void* ws);
bool model_ok(const ec_model* m);
int32_t check_step(const ec_model* m, const ec_state* st, const ec_step_cfg* c, const void* ws);

}  // namespace ec
