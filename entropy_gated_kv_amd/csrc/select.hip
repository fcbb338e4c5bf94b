// Row selection for the next forward pass.
//
// EntropyCache, Chinese summary page §2.2 and Portuguese page §2: a full step
// recomputes every position; a partial step recomputes the still-masked tokens
// of the current block plus the k most recently decoded tokens, taken from a
// decode history of O(k) memory (Chinese page §2.3).  Every other position
// reads its K/V from the cache.
//
// Sliding-window decoding (block_start < 0): the current block is the
// block_len positions from the first masked one, found here on the device, so
// the window moves with the unmasking without a host round trip.  The pages
// name sliding-window decoding among the strategies the method applies to
// (Portuguese page §5, Chinese page §5).
//
// Block diffusion (block_causal): only rows of the current block are ever
// recomputed.  A full step takes the whole block; a partial step its masked
// positions and those of the last k decoded positions that lie inside it (the
// blocks before it are final).  The Chinese page (§5) names block diffusion
// as a place for the entropy signal to drive sub-block recomputation.
//
// One workgroup: the union is marked in an LDS bitmap over [0, L), then
// compacted with a workgroup prefix sum over popcounts, which yields the rows
// in ascending order with duplicates removed.  The same pass can report, for
// each masked position of the block (the LM-head candidates), its index in
// the compact row list.
#include "ec_device.h"
#include "ec_launch.h"

namespace ec {

namespace {

constexpr int kThreads = 1024;

__device__ __forceinline__ int block_exclusive_scan(int v, int* s_wave, int& total) {
  const int lane = threadIdx.x & (kWave - 1), w = threadIdx.x / kWave;
  int incl = v;
#pragma unroll
  for (int o = 1; o < kWave; o <<= 1) {
    const int t = __shfl_up(incl, o, kWave);
    if (lane >= o) incl += t;
  }
  if (lane == kWave - 1) s_wave[w] = incl;
  __syncthreads();
  if (threadIdx.x == 0) {
    int acc = 0;
    for (int k = 0; k < kThreads / kWave; ++k) { const int t = s_wave[k]; s_wave[k] = acc; acc += t; }
    s_wave[kThreads / kWave] = acc;
  }
  __syncthreads();
  total = s_wave[kThreads / kWave];
  return s_wave[w] + incl - v;
}

__global__ __launch_bounds__(kThreads) void select_rows_kernel(
    const int32_t* __restrict__ full_flag, const uint8_t* __restrict__ is_masked, int32_t L,
    int32_t block_start, int32_t block_len, int32_t block_causal, const int32_t* __restrict__ history,
    const int32_t* __restrict__ history_len, int32_t history_cap, int32_t k,
    int32_t* __restrict__ rows, int32_t* __restrict__ n_rows, int32_t* __restrict__ cand_pos,
    int32_t* __restrict__ cand_idx, int32_t* __restrict__ n_cand) {
  extern __shared__ uint32_t bits[];                 // ceil(L / 32) words
  __shared__ int s_wave[kThreads / kWave + 1];
  __shared__ int s_chunk[kThreads];                  // rows before each thread's word run
  __shared__ int s_first;
  const int tid = threadIdx.x;
  const int nwords = (L + 31) / 32;
  const bool full = (*full_flag != 0);
  if (block_start < 0) {
    // sliding window: block_len positions from the first masked one, clipped at L
    if (tid == 0) s_first = L;
    __syncthreads();
    int f = L;
    for (int p = tid; p < L; p += kThreads)
      if (is_masked[p]) { f = p; break; }
    atomicMin(&s_first, f);
    __syncthreads();
    block_start = s_first;
    block_len = min(block_len, L - block_start);
  }
  const int bend = block_start + block_len;
  // the positions a step may recompute: all of them, or the current block
  const int lo = block_causal ? block_start : 0, hi = block_causal ? bend : L;

  if (full) {
    for (int p = lo + tid; p < hi; p += kThreads) rows[p - lo] = p;
    if (tid == 0) *n_rows = hi - lo;
  } else {
    for (int w = tid; w < nwords; w += kThreads) bits[w] = 0u;
    __syncthreads();
    for (int p = block_start + tid; p < bend; p += kThreads)
      if (is_masked[p]) atomicOr(&bits[p >> 5], 1u << (p & 31));
    const int hl = *history_len;
    const int kk = min(k, hl);
    for (int j = tid; j < kk; j += kThreads) {
      const int p = history[(hl - kk + j) % history_cap];
      if (p >= lo && p < hi) atomicOr(&bits[p >> 5], 1u << (p & 31));
    }
    __syncthreads();
    // Each thread owns a contiguous run of words, so ranks come out ascending.
    const int per = (nwords + kThreads - 1) / kThreads;
    const int w0 = min(nwords, tid * per), w1 = min(nwords, w0 + per);
    int cnt = 0;
    for (int w = w0; w < w1; ++w) cnt += __popc(bits[w]);
    int total;
    int pos = block_exclusive_scan(cnt, s_wave, total);
    s_chunk[tid] = pos;
    for (int w = w0; w < w1; ++w) {
      uint32_t b = bits[w];
      while (b) {
        const int bit = __ffs(b) - 1;
        b &= b - 1;
        rows[pos++] = w * 32 + bit;
      }
    }
    if (tid == 0) *n_rows = total;
  }

  if (cand_pos != nullptr) {
    // Candidates = masked positions of the block, ascending; their index in rows.
    __syncthreads();
    const int per = (nwords + kThreads - 1) / kThreads;
    const int p = block_start + tid;                // block_len <= kThreads (checked on host)
    const bool is_c = (tid < block_len) && is_masked[p];
    int total;
    const int slot = block_exclusive_scan(is_c ? 1 : 0, s_wave, total);
    if (is_c) {
      int rank;
      if (full) {
        rank = p - lo;
      } else {
        const int wp = p >> 5;
        const int owner = wp / per;
        rank = s_chunk[owner];
        for (int w = owner * per; w < wp; ++w) rank += __popc(bits[w]);
        rank += __popc(bits[wp] & ((1u << (p & 31)) - 1u));
      }
      cand_pos[slot] = p;
      cand_idx[slot] = rank;
    }
    if (tid == 0) *n_cand = total;
  }
}

}  // namespace

int32_t select_max_L() { return kSelectMaxL; }

hipError_t launch_select_rows(const int32_t* full_flag, const uint8_t* is_masked, int32_t L,
                              int32_t block_start, int32_t block_len, int32_t block_causal,
                              const int32_t* history, const int32_t* history_len,
                              int32_t history_cap, int32_t k, int32_t* rows, int32_t* n_rows,
                              int32_t* cand_pos, int32_t* cand_idx, int32_t* n_cand,
                              hipStream_t s) {
  const size_t lds = size_t((L + 31) / 32) * sizeof(uint32_t);
  hipLaunchKernelGGL(select_rows_kernel, dim3(1), dim3(kThreads), lds, s, full_flag, is_masked, L,
                     block_start, block_len, block_causal, history, history_len, history_cap, k,
                     rows, n_rows, cand_pos, cand_idx, n_cand);
  return hipGetLastError();
}

}  // namespace ec
