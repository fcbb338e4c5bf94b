/*
 * ec.h -- C ABI of the EntropyCache denoising-step library (libec.so, gfx950).
 *
 * One EntropyCache denoising step (paper "EntropyCache: Decoded Token Entropy
 * Guided KV Caching for Diffusion Language Models"; Chinese summary page
 * gist.science/zh/paper/2603.18489, technical summary §2.2, algorithm
 * workflow) has three phases: a forward pass that is full or partial according
 * to the previous step's flag, decoding plus the maximum entropy of the newly
 * decoded tokens, and the threshold decision that sets the next step's flag.
 * The entry points below are those phases and the kernels inside them.
 *
 * Conventions shared by every entry point
 *  - Tensor arguments are DEVICE pointers, allocated and owned by the caller.
 *    The library never allocates or frees device memory; scratch space is a
 *    caller-provided workspace sized by the matching *_workspace_bytes().
 *  - Work is enqueued on the caller's stream and the call returns at once; no
 *    call synchronises the device or reads device memory on the host.  Row
 *    counts and decision flags that live in device memory stay there.
 *  - Every call returns an ec_status.  All argument checks run on the host
 *    before anything is enqueued, and nothing is enqueued on an error.
 *  - Tensor pointers must be 16-byte aligned and row strides multiples of 16
 *    bytes (EC_E_ALIGN otherwise).
 *  - dtype is EC_F32 or EC_BF16 for activations, weights, caches and logits of
 *    one call.  Entropies, maxima and probabilities are always float32.
 *  - The library keeps no global mutable state; calls on different streams
 *    with disjoint buffers may run concurrently.
 */
#ifndef EC_H_
#define EC_H_

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum ec_status {
  EC_OK = 0,
  EC_E_NULL = -1,        /* a required pointer is NULL                        */
  EC_E_SHAPE = -2,       /* a size is out of range or inconsistent             */
  EC_E_DTYPE = -3,       /* unknown dtype                                      */
  EC_E_WORKSPACE = -4,   /* workspace smaller than *_workspace_bytes()         */
  EC_E_ALIGN = -5,       /* pointer or stride not 16-byte aligned              */
  EC_E_LAUNCH = -6,      /* the HIP runtime refused a launch                   */
  EC_E_UNSUPPORTED = -7  /* a valid but unsupported combination (e.g. head dim) */
} ec_status;

enum { EC_F32 = 0, EC_BF16 = 1 };

/* Static description of a status code (never NULL). */
const char* ec_status_string(int32_t status);

/* ABI revision of this header; bumped on any signature or struct change. */
int32_t ec_abi_version(void);
#define EC_ABI_VERSION 6

/* --------------------------------------------------------------------------
 * Entropy pass (a1) and decision (a2).
 *
 * Source: EntropyCache Chinese summary page, §2.2: E_{t+1} is the largest
 * softmax entropy -sum_j p_ij ln p_ij over the newly decoded tokens i, and
 * E_{t+1} > tau sends the next step to a full forward, E_{t+1} <= tau to a
 * partial one; §2.3: the decision costs O(V) compute.  The Portuguese page
 * (gist.science/pt/paper/2603.18489, §2) states the same strict ">" rule.
 *
 * For each row r < n_rows of logits [n_rows, row_stride] (dtype elements,
 * first V of each row used):
 *   row_entropy[r] = H = -sum_j p_j ln p_j with p = softmax(row) (nats)
 *   row_argmax[r]  = lowest j with row[j] = max (NaN ignored; all-NaN -> 0)
 *   row_top1[r]    = max_j p_j
 * then over the decoded rows D:
 *   *e_max     = max_{r in D} H_r   (-inf if D is empty, NaN if any H_r is NaN)
 *   *full_flag = (*e_max > tau) || isnan(*e_max)
 * -inf logits contribute p = 0.  A row containing NaN or +inf has H = NaN and
 * p1 = NaN; an all -inf row has H = p1 = NaN.
 *
 * D is decoded_rows[0 .. *n_decoded) (device int32 indices into the rows,
 * each < n_rows; *n_decoded <= max_decoded), or every row when decoded_rows
 * is NULL (then n_decoded is ignored).
 *
 * Determinism: the per-row results depend only on that row's V logits (the
 * split of V into segments depends on V alone), so they are bitwise identical
 * whatever n_rows, D or the other rows are.
 *
 * row_argmax and row_top1 may be NULL.  ws must hold
 * ec_entropy_workspace_bytes(n_rows, V) bytes (16-byte aligned); it holds
 * per-segment partial statistics.  Two calls that overlap in time must not
 * share a workspace.
 * Errors: EC_E_NULL (logits, row_entropy, e_max, full_flag or ws NULL),
 * EC_E_SHAPE (n_rows < 1, V < 1, row_stride < V, max_decoded < 0),
 * EC_E_DTYPE, EC_E_ALIGN, EC_E_WORKSPACE, EC_E_LAUNCH.
 * ------------------------------------------------------------------------ */
size_t ec_entropy_workspace_bytes(int64_t n_rows, int64_t V);

int32_t ec_entropy_max(const void* logits, int32_t dtype, int64_t n_rows, int64_t V,
                       int64_t row_stride,
                       const int32_t* decoded_rows, const int32_t* n_decoded, int32_t max_decoded,
                       float tau,
                       float* row_entropy, int32_t* row_argmax, float* row_top1,
                       float* e_max, int32_t* full_flag,
                       void* ws, size_t ws_bytes, hipStream_t stream);

/* --------------------------------------------------------------------------
 * Entropy pass and decision with no workspace, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation).
 *
 * Same arguments (minus ws / ws_bytes), kernels and results, bit for bit, as
 * ec_entropy_max above.  The per-segment partial statistics live in a static
 * device array of EC_NOALLOC_SCRATCH_BYTES that each GPU the library runs on
 * holds until the process ends; the call allocates nothing.  Its device
 * address is looked up on the stream's device at that device's first call.
 * Calls on one GPU share the array: two calls that overlap in time on the
 * same GPU race (serialise them, for example on one stream).  Nothing in the
 * array needs clearing between calls.
 * Limit: the partial statistics, n_rows * ceil(V / 4096) * 16 bytes (bf16)
 * or n_rows * ceil(V / 2048) * 16 bytes (fp32), must fit in
 * EC_NOALLOC_SCRATCH_BYTES (8 MiB: e.g. 4096 rows of V = 126464 in bf16 use
 * 2 MiB); a larger call returns EC_E_WORKSPACE before anything is enqueued.
 * Errors: as ec_entropy_max; EC_E_LAUNCH also when the array's device address
 * cannot be looked up on the stream's device.
 * ------------------------------------------------------------------------ */
#define EC_NOALLOC_SCRATCH_BYTES (8u << 20)

int32_t ec_entropy_max_noalloc(const void* logits, int32_t dtype, int64_t n_rows, int64_t V,
                               int64_t row_stride,
                               const int32_t* decoded_rows, const int32_t* n_decoded,
                               int32_t max_decoded, float tau,
                               float* row_entropy, int32_t* row_argmax, float* row_top1,
                               float* e_max, int32_t* full_flag, hipStream_t stream);

/* --------------------------------------------------------------------------
 * Row selection (a3).
 *
 * Source: EntropyCache Chinese page §2.2 and Portuguese page §2: a full step
 * recomputes every position; a partial step recomputes only the still-masked
 * tokens and the k most recently decoded tokens, kept in a decode history
 * (O(k) memory, Chinese page §2.3); all other positions read the KV cache.
 *
 *   *full_flag != 0:  rows = 0, 1, ..., L-1
 *   *full_flag == 0:  rows = ascending union of
 *                       { p in [block_start, block_start+block_len) : is_masked[p] }
 *                     and the last min(k, *history_len) entries of the history
 *
 * history is a ring of history_cap device int32 positions: entry i (the i-th
 * position ever decoded, 0-based) is at history[i % history_cap]; *history_len
 * is the total count appended.  Requires k <= history_cap.  Positions must be
 * < L; duplicates in the union are written once.
 * Sliding-window decoding: block_start = -1 makes the block the block_len
 * positions from the first masked position, clipped at L (empty when nothing
 * is masked), found on the device (Portuguese page §5 and Chinese page §5 name
 * sliding-window decoding among the strategies the method applies to).
 * Block diffusion: block_causal = 1 restricts both sets to the current block
 * (the blocks before it are final): a full step selects
 *   rows = block_start, ..., block_start + block_len - 1
 * and a partial step the block's masked positions plus those of the last
 * min(k, *history_len) history entries that lie inside the block.  The
 * Chinese page (§5, generality) names block diffusion as a place for the
 * entropy signal to drive sub-block recomputation; the step runs such blocks
 * with block-causal attention (ec_step_cfg.block_causal).
 * Outputs: rows [L] (device, first *n_rows valid) and *n_rows (device).
 * Errors: EC_E_NULL, EC_E_SHAPE (L < 1, block outside [0, L), block_start < -1,
 * block_len > L, k < 0, k > history_cap, history_cap < 1, block_causal not 0
 * or 1, block_causal with block_start = -1), EC_E_LAUNCH.
 * ------------------------------------------------------------------------ */
int32_t ec_select_rows(const int32_t* full_flag, const uint8_t* is_masked, int32_t L,
                       int32_t block_start, int32_t block_len, int32_t block_causal,
                       const int32_t* history, const int32_t* history_len, int32_t history_cap,
                       int32_t k, int32_t* rows, int32_t* n_rows, hipStream_t stream);

/* --------------------------------------------------------------------------
 * Selective KV refresh (a4).
 *
 * Source: EntropyCache Chinese page §2.2 (a partial pass recomputes K/V only
 * for the selected rows, the rest is read from the cache) and Portuguese page
 * §2 (the full pass refreshes the whole KV cache).
 *
 * For r < *n_rows (device count, <= max_rows):
 *   y_r = x[r, :] . W^T        (W = w_qkv [(Hq + 2 Hkv) * dh, d], row-major,
 *                               output features ordered Q heads, K heads, V heads)
 *   q_out[r, h, :]               = y_r[h*dh : (h+1)*dh]                 h < Hq
 *   k_cache[g, rows[r], :]       = y_r[(Hq+g)*dh : ...]                 g < Hkv
 *   v_cache[g, :, rows[r]]       = y_r[(Hq+Hkv+g)*dh : ...]             g < Hkv
 * Layouts: x [max_rows, x_stride] (x_stride >= d), q_out [max_rows, Hq, dh],
 * k_cache [Hkv, L_cap, dh], v_cache [Hkv, dh, L_cap] (V is stored transposed
 * so that the attention's P.V contraction reads contiguous positions).
 * Cache rows not listed in rows[] are left untouched.  Accumulation is fp32;
 * outputs are rounded to dtype (nearest even).  rows[r] < L_cap, distinct.
 * ws holds split-K partial sums: ec_kv_refresh_workspace_bytes(...) bytes
 * (may be 0, then ws may be NULL).
 * Supported: d a multiple of 128 (bf16) or 64 (fp32), dh in {32, 64, 128},
 * Hq % Hkv == 0.
 * Errors: EC_E_NULL, EC_E_SHAPE, EC_E_DTYPE, EC_E_ALIGN, EC_E_WORKSPACE,
 * EC_E_UNSUPPORTED, EC_E_LAUNCH.
 * ------------------------------------------------------------------------ */
size_t ec_kv_refresh_workspace_bytes(int32_t max_rows, int32_t d, int32_t Hq, int32_t Hkv,
                                     int32_t dh, int32_t dtype);

int32_t ec_kv_refresh(const void* x, int64_t x_stride, const int32_t* rows, const int32_t* n_rows,
                      int32_t max_rows, const void* w_qkv, int32_t d, int32_t Hq, int32_t Hkv,
                      int32_t dh, int32_t dtype, void* q_out, void* k_cache, void* v_cache,
                      int32_t L_cap, void* ws, size_t ws_bytes, hipStream_t stream);

/* --------------------------------------------------------------------------
 * Bidirectional attention of the selected rows against the whole cache (a5).
 *
 * Source: EntropyCache Portuguese page §1 and Chinese page §1: diffusion LMs
 * use bidirectional attention, so every position attends to every position
 * (no causal mask); the selected rows' queries read all L cache rows, fresh or
 * stale.  The split of the cache into partitions merged by log-sum-exp follows
 * the split-KV kernel described on the Prefilling-dLLM page
 * (gist.science/pt/paper/2606.10537, attention-kernel section).
 *
 * For r < *n_rows, h < Hq, g = h / (Hq / Hkv):
 *   out[r, h, :] = softmax_j( scale * q[r, h, :] . K[g, j, :] ) . V[g, j, :],  j < L
 * with K = k_cache [Hkv, L_cap, dh] and V stored transposed, v_cache
 * [Hkv, dh, L_cap].  fp32 accumulation, output rounded to dtype.
 * q [max_rows, Hq, dh], out [max_rows, Hq, dh].  1 <= L <= L_cap.
 * ws must hold ec_attention_workspace_bytes(max_rows, L, Hq, Hkv, dh).
 * Supported: dh in {32, 64, 128}, Hq % Hkv == 0, Hq / Hkv <= 16.
 * Errors: EC_E_NULL, EC_E_SHAPE, EC_E_DTYPE, EC_E_ALIGN, EC_E_WORKSPACE,
 * EC_E_UNSUPPORTED, EC_E_LAUNCH.
 * ------------------------------------------------------------------------ */
size_t ec_attention_workspace_bytes(int32_t max_rows, int32_t L, int32_t Hq, int32_t Hkv,
                                    int32_t dh);

int32_t ec_bidir_attention(const void* q, const int32_t* n_rows, int32_t max_rows,
                           const void* k_cache, const void* v_cache, int32_t L, int32_t L_cap,
                           int32_t Hq, int32_t Hkv, int32_t dh, float scale, int32_t dtype,
                           void* out, void* ws, size_t ws_bytes, hipStream_t stream);

/* --------------------------------------------------------------------------
 * One full denoising step (all of the above plus the glue around them).
 *
 * Source: EntropyCache Chinese page §2.2 (the three phases of a step) and
 * Portuguese page §2 (decode, skip-or-recompute decision, decode history).
 *
 * Sequence per call, all on `stream`, no host synchronisation:
 *   rows   = select(*full_flag, is_masked, current block, history, k)
 *   x      = tok_emb[tokens[rows]] + pos_emb[rows]
 *   per layer: [a = rmsnorm(x) * norm_attn] ; refresh Q/K/V of rows ;
 *              o = attention(Q, whole cache) ; x += o . W_o^T ;
 *              [a2 = rmsnorm(x) * norm_ffn ; x += (silu(a2 W_gate^T) * a2 W_up^T) . W_down^T]
 *   [x = rmsnorm(x) * norm_final]
 *   cand   = masked positions of the current block (ascending)
 *   logits[i, :] = (x[cand_i] . W_lm^T) * logit_scale[cand_i]
 *   per candidate: H, argmax, p1 (as ec_entropy_max)
 *   chosen = the min(n_unmask, |cand|) candidates of largest p1 (ties -> lower position)
 *   tokens[c] = argmax_c, is_masked[c] = 0 for c in chosen;
 *   chosen positions appended to the history ring in ascending order
 *   *e_max = max H over chosen (-inf if none); *full_flag = (*e_max > tau) || isnan
 * Without an LM head (model->w_lm == NULL) the caller decodes: before the call
 * it writes the logits of the n_unmask rows it decoded this step into
 * state->logits ([n_unmask, V], 1 <= n_unmask <= block_len); the step then runs
 * select, embed and the layers as above and ends with
 *   H, argmax, p1 of those rows; *e_max = max H over all of them;
 *   *full_flag = (*e_max > tau) || isnan
 * leaving tokens, is_masked, history, chosen and n_chosen untouched and
 * skipping the final norm (nothing reads it).  This is the steady-state
 * long-context step, where the decoded rows come from outside the layer.
 * The first step of a sequence must run with *full_flag = 1 (no cache yet).
 * ws (ec_step_workspace_bytes(model, max_block) bytes) is scratch: every
 * region is written before it is read, so no initial contents are required.
 * Norms and FFN are present iff d_ffn > 0.  d, Hq*dh and d_ffn must be
 * multiples of 128 (bf16) or 64 (fp32), and V of 32 when w_lm is given
 * (EC_E_UNSUPPORTED otherwise); block_len is at most 1024.  The block (block_start,
 * block_len) and n_unmask are host values: the schedule is fixed on the host.
 * ------------------------------------------------------------------------ */
typedef struct ec_layer {
  const void* w_qkv;      /* [(Hq + 2 Hkv) * dh, d]                      */
  const void* w_o;        /* [d, Hq * dh]                                */
  const void* norm_attn;  /* [d] (d_ffn > 0 only, else NULL)             */
  const void* norm_ffn;   /* [d] (d_ffn > 0 only)                        */
  const void* w_gate;     /* [d_ffn, d] (d_ffn > 0 only)                 */
  const void* w_up;       /* [d_ffn, d] (d_ffn > 0 only)                 */
  const void* w_down;     /* [d, d_ffn] (d_ffn > 0 only)                 */
} ec_layer;

typedef struct ec_model {
  int32_t n_layers, d, Hq, Hkv, dh, d_ffn, V, L_cap, dtype;
  float rms_eps;
  const void* tok_emb;        /* [V + 1, d]; row V is the MASK embedding   */
  const void* pos_emb;        /* [L_cap, d]                                */
  const ec_layer* layers;     /* host array [n_layers]                     */
  const void* norm_final;     /* [d] (d_ffn > 0 only)                      */
  const void* w_lm;           /* [V, d], or NULL: no LM head (see above)   */
  const float* logit_scale;   /* [L_cap] device float32, or NULL (= 1)     */
  /* Optional: w_lm repacked by ec_pack_lm_head, or NULL.  When set (bf16,
   * V % 16 == 0, 16-byte aligned), the LM head of steps whose block holds at
   * most 32 positions reads it instead of w_lm if V > 32704 and d % 256 == 0
   * (same arithmetic, same bits); w_lm must still be given. */
  const void* w_lm_packed;
} ec_model;

typedef struct ec_state {
  int32_t L;                  /* sequence length, <= L_cap                 */
  int32_t* tokens;            /* [L] device                                */
  uint8_t* is_masked;         /* [L] device                                */
  int32_t* history;           /* [history_cap] device ring                 */
  int32_t* history_len;       /* [1] device                                */
  int32_t history_cap;
  int32_t* full_flag;         /* [1] device: read as this step's mode, then
                                 overwritten with the next step's decision */
  void* const* k_cache;       /* host array [n_layers] of [Hkv, L_cap, dh] */
  void* const* v_cache;       /* host array [n_layers] of [Hkv, dh, L_cap] */
  /* per-step outputs (device, caller-owned) */
  int32_t* rows;              /* [L_cap]                                   */
  int32_t* n_rows;            /* [1]                                       */
  /* [max_block, V] dtype.  May be NULL with an LM head whose packed copy the
   * step reads (w_lm_packed set, block_len <= 32, V > 32704, d % 256 == 0;
   * EC_E_UNSUPPORTED otherwise, EC_E_NULL without w_lm_packed): the LM head
   * then writes no logits but each candidate's softmax statistics per group
   * of column tiles (in the workspace), which the step folds into H, argmax
   * and p1 in place of the entropy pass.  Every other output is as with a
   * buffer; H, p1 and E may differ from it in the last float32 bits (the
   * statistics are summed in another order). */
  void* logits;
  float* row_entropy;         /* [max_block]                               */
  int32_t* row_argmax;        /* [max_block]                               */
  float* row_top1;            /* [max_block]                               */
  int32_t* chosen;            /* [max_block] positions, ascending          */
  int32_t* n_chosen;          /* [1]                                       */
  float* e_max;               /* [1]                                       */
  /* Optional diagnostic, or NULL: [n_layers][2] device float32.  On a full
   * step, layer l's entries become the mean and the maximum over positions
   * p < L of 1 - cos(stale_p, fresh_p), where stale_p / fresh_p are position
   * p's Value vector (concatenated over the KV heads) before and after the
   * step's refresh; positions with an all-zero vector are left out (NaN when
   * none is left).  Partial steps leave it unchanged.  EntropyCache, Chinese
   * summary page §2.1 and Portuguese page §2: the entropy of decoded tokens
   * tracks this drift of the Value vectors.  Needs 16-byte aligned caches. */
  float* kv_drift;
  /* Optional observation point, or NULL: [L_cap, Hq, dh] device, the model's
   * dtype, 16-byte aligned.  After the step, rows [0, *n_rows) hold the last
   * layer's attention output for the selected rows, in selection order (the
   * bidirectional attention of Portuguese page §1 / Chinese page §1, before
   * the output projection).  One extra device-to-device copy per step. */
  void* attn_out;
} ec_state;

/* Step modes (ec_step_cfg.mode).  EC_MODE_DEVICE: the mode is read from
 * *full_flag on the device and the kernels of both modes are launched (those
 * of the other mode exit at once), so the host never waits.  EC_MODE_FULL /
 * EC_MODE_PARTIAL: the caller states what *full_flag holds (having read it
 * after the previous step) and only that mode's kernels are launched, which
 * saves one launch per GEMM and per attention call.  A statement that differs
 * from *full_flag leaves the step's results undefined (every access stays in
 * bounds). */
enum { EC_MODE_DEVICE = 0, EC_MODE_FULL = 1, EC_MODE_PARTIAL = 2 };

typedef struct ec_step_cfg {
  float tau;
  int32_t k;
  int32_t n_unmask;
  int32_t block_start;        /* or -1: sliding window (see ec_select_rows) */
  int32_t block_len;          /* <= max_block of the workspace             */
  int32_t mode;               /* EC_MODE_* (EC_E_SHAPE otherwise)          */
  /* 1: block diffusion.  Rows are selected inside the current block only
   * (ec_select_rows with block_causal = 1) and attend to the keys at
   * positions [0, block_start + block_len): attention is block-causal, the
   * blocks before the current one being final.  A finished block is made
   * final by one step with *full_flag set to 1 and n_unmask = 0 (a full pass
   * over its rows that decodes nothing; it leaves *full_flag = 0).
   * Requires block_start >= 0.  Chinese page §5 (generality): entropy as the
   * recompute signal for sub-blocks in block diffusion. */
  int32_t block_causal;
} ec_step_cfg;

/* Optional per-phase timing: when non-NULL, phase_events holds 2*EC_PHASE_COUNT
 * event handles and ec_step records events[2*i] and events[2*i+1] around
 * phase i on the stream.  Per-layer phases (QKV, attention, O-projection, FFN)
 * are bracketed in the first layer only.  A NULL entry skips that record, so a
 * caller can time one phase without recording events around the others. */
enum {
  EC_PHASE_SELECT = 0, EC_PHASE_EMBED, EC_PHASE_QKV, EC_PHASE_ATTN, EC_PHASE_OPROJ,
  EC_PHASE_FFN, EC_PHASE_LMHEAD, EC_PHASE_ENTROPY, EC_PHASE_DECIDE, EC_PHASE_COUNT
};

/* Repack the LM-head weight for streaming (an optional, one-time step at
 * model load).  w_lm [V, d] bf16 row-major becomes, for each group of 16
 * rows, its d / 32 blocks of 16 rows x 32 columns in column order; a block is
 * 1 KB: entry (row n, columns 8g .. 8g + 7) of the block is its 16-byte
 * chunk 16 g + n.  The LM head's loads then read each 8 KB of a group's
 * weights from consecutive addresses.  The logits are those of w_lm (the
 * LM head of Chinese page §2.2's forward pass; the layout changes only where
 * the weights are read from).
 * w_packed: device, V * d bf16 elements, caller-owned, 16-byte aligned, not
 * overlapping w_lm.  Asynchronous on the stream.
 * Errors: EC_E_NULL, EC_E_DTYPE (not bf16), EC_E_SHAPE (V < 16, V % 16 != 0,
 * d < 32, d % 32 != 0), EC_E_UNSUPPORTED (V * d > 2^40), EC_E_ALIGN,
 * EC_E_LAUNCH. */
int32_t ec_pack_lm_head(const void* w_lm, int32_t V, int32_t d, int32_t dtype, void* w_packed,
                        hipStream_t stream);

size_t ec_step_workspace_bytes(const ec_model* model, int32_t max_block);

int32_t ec_step(const ec_model* model, const ec_state* state, const ec_step_cfg* cfg,
                void* ws, size_t ws_bytes, hipEvent_t* phase_events, hipStream_t stream);

#ifdef __cplusplus
}
#endif
#endif /* EC_H_ */
