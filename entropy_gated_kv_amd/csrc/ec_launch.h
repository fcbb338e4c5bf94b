// Host-side launchers of the gfx950 kernels, called by the C-ABI layer after
// its argument checks.  Internal to libec.so.
#pragma once
#include <hip/hip_runtime_api.h>
#include <stddef.h>
#include <stdint.h>

#include "ec_limits.h"

namespace ec {

// ---- entropy pass ----------------------------------------------------------
struct EntropyPartial {   // online softmax statistics of one V segment
  float m;                // max over the segment (+/-inf possible)
  float z;                // sum 2^u, u = (x - m) log2(e)
  float s2;               // sum 2^u * u
  int32_t idx;            // lowest index holding m (INT32_MAX: none)
};
// Rows are split into segments of 512 16-byte vectors (4096 bf16 / 2048 fp32).
int entropy_segments(int64_t V, int dtype);
size_t entropy_ws_bytes(int64_t n_rows, int64_t V, int dtype);

// Per-row H / argmax / p1 for rows < min(n_rows, *n_rows_dev) (n_rows_dev may
// be NULL) and, when e_max != NULL, E = max over D of H and flag = E > tau
// (NaN -> 1); D NULL means rows [0, n_rows).  ws holds the segment partials.
int device_cu_count();
// The entropy pass of a step's few rows (at most step_max_rows()) and its
// decision: partials, then one workgroup that folds each row and decides.
// cand_pos != NULL: rows are the block's candidates at positions cand_pos
// (*n_rows_dev of them); the n_unmask of largest p1 are unmasked, decoded,
// appended to the history, E = max H over them.  cand_pos == NULL: E = max H
// over all max_rows rows (n_rows_dev NULL); nothing else is written.
// Then *flag = (E > tau) || isnan(E).
int32_t step_max_rows();
// The same decode and decision from partials the packed LM head wrote in its
// epilogue (GemmArgs::stats): P per row, row r's at part[r * P ...], at most
// kLmStatRows rows; the logits are not read.
hipError_t launch_entropy_step_fused(const EntropyPartial* part, int32_t P, int32_t max_rows,
                                     const int32_t* n_rows_dev, float* H, int32_t* argmax, float* p1,
                                     const int32_t* cand_pos, int32_t n_unmask, float tau,
                                     int32_t* chosen, int32_t* n_chosen, int32_t* tokens,
                                     uint8_t* is_masked, int32_t* history, int32_t* history_len,
                                     int32_t history_cap, float* e_max, int32_t* flag, hipStream_t s);
hipError_t launch_entropy_step(const void* logits, int dtype, int32_t max_rows,
                               const int32_t* n_rows_dev, int64_t V, int64_t stride, float* H,
                               int32_t* argmax, float* p1, const int32_t* cand_pos,
                               int32_t n_unmask, float tau, int32_t* chosen, int32_t* n_chosen,
                               int32_t* tokens, uint8_t* is_masked, int32_t* history,
                               int32_t* history_len, int32_t history_cap, float* e_max,
                               int32_t* flag, void* ws, hipStream_t s);
hipError_t launch_entropy(const void* logits, int dtype, int64_t n_rows, const int32_t* n_rows_dev,
                          int64_t V, int64_t stride, float* H, int32_t* argmax, float* p1,
                          const int32_t* D, const int32_t* nD, int32_t maxD, float tau,
                          float* e_max, int32_t* flag, void* ws, hipStream_t s);

}  // namespace ec

namespace ec {

// ---- row selection -----------------------------------------------------------
int32_t select_max_L();
hipError_t launch_select_rows(const int32_t* full_flag, const uint8_t* is_masked, int32_t L,
                              int32_t block_start, int32_t block_len, int32_t block_causal,
                              const int32_t* history, const int32_t* history_len,
                              int32_t history_cap, int32_t k, int32_t* rows, int32_t* n_rows,
                              int32_t* cand_pos, int32_t* cand_idx, int32_t* n_cand,
                              hipStream_t s);

// ---- glue --------------------------------------------------------------------
hipError_t launch_embed(int dtype, const void* tok_emb, const void* pos_emb, const int32_t* tokens,
                        const int32_t* rows, const int32_t* n_rows, int max_rows, int d, void* x,
                        hipStream_t s);
hipError_t launch_rmsnorm(int dtype, const void* x, const int32_t* n_rows, int max_rows, int d,
                          const void* gain, float eps, void* out, hipStream_t s);


// ---- row GEMM with fused epilogues ---------------------------------------------
// C[r, n] = sum_k A[row(r), k] * W[n, k] for r < *n_rows_dev (<= max_rows), n < N,
// where row(r) = a_idx ? a_idx[r] : r.  W is [N, K] row-major.
enum class Epi : int {
  kStore = 0,     // C[r, n] = acc                                    (C [max_rows, ldc])
  kQKV = 1,       // Q / K cache / V^T cache scatter at rows[r]
  kResidual = 2,  // C[r, n] = C[r, n] + acc  (in place)
  kSwiGLU = 3,    // C[r, n] = silu(acc) * acc2, acc2 from W2
  kLogits = 4,    // C[r, n] = acc * scale[scale_pos[r]]  (scale may be NULL)
};
// Launch paths of the row-count-dependent operations: device row counts up
// to kSmallMaxRows (skinny GEMM, split-KV attention) or above (tiled GEMM,
// unsplit attention).
constexpr unsigned kPathSmall = 1u, kPathLarge = 2u;

struct GemmArgs {
  int dtype = 0;
  Epi epi = Epi::kStore;
  const void* A = nullptr;
  int64_t lda = 0;
  const int32_t* a_idx = nullptr;
  const int32_t* n_rows_dev = nullptr;
  int max_rows = 0;
  // Optional tighter bound on the device row count whenever that count is at
  // most 128 (the rows the skinny kernel takes); 0 = max_rows.  The caller
  // guarantees it: rows past the bound would be left unwritten.
  int skinny_rows = 0;
  // Kernels to launch: kPathSmall (skinny kernel and its split-K reduction,
  // device row counts <= 128) and/or kPathLarge (tiled kernel, counts > 128).
  // Each exits at once on a count outside its range; a caller that knows the
  // count's range may leave the other out.
  unsigned paths = kPathSmall | kPathLarge;
  const void* W = nullptr;
  const void* W2 = nullptr;
  // kLogits, bf16: W in the fragment layout (launch_pack_fragments), or null;
  // the packed LM-head kernel then reads it instead of W
  const void* W_packed = nullptr;
  int N = 0, K = 0;
  void* C = nullptr;
  int64_t ldc = 0;
  // kQKV
  const int32_t* rows = nullptr;
  void* q_out = nullptr;
  void* k_cache = nullptr;
  void* v_cache = nullptr;
  int Hq = 0, Hkv = 0, dh = 0, L_cap = 0;
  // kLogits
  const float* scale = nullptr;
  const int32_t* scale_pos = nullptr;
  // kLogits, optional: where the packed LM-head kernel may also write each
  // row's softmax statistics, one partial per group of column tiles in column
  // order (row r's at stats[r * groups ...]; at most kLmStatRows rows times
  // lmhead_max_stat_groups(N) partials).  The launcher sets *stats_groups (a
  // host int) to the groups per row when it did, else to 0.
  EntropyPartial* stats = nullptr;
  int* stats_groups = nullptr;
};
// The most partials per row the packed LM head writes for N columns.
int lmhead_max_stat_groups(int N);
size_t gemm_ws_bytes(const GemmArgs& a);
// Reduction dimensions (d, Hq*dh, d_ffn) must be multiples of this (128 bf16, 64 fp32).
int gemm_k_multiple(int dtype);
hipError_t launch_gemm_rows(const GemmArgs& a, void* ws, hipStream_t s);
// Repack a bf16 [N, K] weight (N % 16 == 0, K % 32 == 0) into the fragment
// layout read by the packed LM-head kernel; out holds N * K elements.
hipError_t launch_pack_fragments(const void* W, int64_t N, int64_t K, void* out, hipStream_t s);

// ---- KV drift of a full step (diagnostic) ------------------------------------------
// Workspace: a copy of one layer's transposed Value cache [nrow = Hkv * dh, L_cap]
// plus L_cap floats.  Both launches exit at once unless *flag (the step's mode) is 1.
size_t value_drift_ws_bytes(int dtype, int nrow, int L_cap);
// Before the layer's refresh: copy columns [0, L) of the Value cache into ws.
hipError_t launch_value_drift_snapshot(int dtype, const int32_t* flag, const void* v_cache, int nrow,
                                       int L, int L_cap, void* ws, hipStream_t s);
// After it: out[0] = mean, out[1] = max over positions of 1 - cos(stale, fresh).
hipError_t launch_value_drift(int dtype, const int32_t* flag, const void* v_cache, int nrow, int L,
                              int L_cap, void* ws, float* out, hipStream_t s);

// ---- bidirectional attention -----------------------------------------------------
struct AttnArgs {
  int dtype = 0;
  const void* q = nullptr;            // [max_rows, Hq, dh]
  const int32_t* n_rows_dev = nullptr;
  int max_rows = 0;
  const void* k_cache = nullptr;      // [Hkv, L_cap, dh]
  const void* v_cache = nullptr;      // [Hkv, dh, L_cap]
  int L = 0, L_cap = 0, Hq = 0, Hkv = 0, dh = 0;
  float scale = 1.f;
  void* out = nullptr;                // [max_rows, Hq, dh]
  // kPathSmall: split-KV kernel and merge (<= 128 rows); kPathLarge: unsplit
  // kernel (> 128 rows), as for GemmArgs.
  unsigned paths = kPathSmall | kPathLarge;
  // Optional tighter bound on the device row count whenever that count is at
  // most 128 (the split-KV plan is made for it); 0 = max_rows.  The caller
  // guarantees it.
  int small_rows = 0;
};
size_t attn_ws_bytes(int max_rows, int L, int Hq, int Hkv, int dh);
hipError_t launch_attention(const AttnArgs& a, void* ws, hipStream_t s);

}  // namespace ec
