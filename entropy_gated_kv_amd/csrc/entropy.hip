// Entropy pass: per-row softmax entropy, argmax and top-1 probability in one
// HBM stream over the logits, then the maximum over the decoded rows and the
// threshold decision.
//
// EntropyCache, Chinese summary page §2.2: E_{t+1} = max over the newly
// decoded tokens of -sum_j p_ij ln p_ij, and E_{t+1} > tau triggers a full
// recompute; §2.3: the decision is O(V) per token.  Portuguese page §2: the
// same strict ">" rule.
//
// Statistics: for a run of logits x with maximum m,
//   z = sum 2^u,  s2 = sum 2^u u,  u = (x - m) log2 e,
// give H = ln 2 (log2 z - s2 / z) and p1 = 1 / z.  Two runs merge exactly by
// rescaling to the larger maximum (see merge()).
//
// Work decomposition (a function of V only, so every per-row result is a
// fixed function of that row's logits, whatever the batch):
//   * a row is cut into segments of 512 16-byte vectors (4096 bf16 or 2048
//     fp32 elements), one wave per segment, four independent waves per
//     workgroup;
//   * lane l owns the vectors l, l+64, ..., (8 in a full segment), all loaded
//     before any arithmetic, so a wave keeps 8 KB in flight and the many
//     resident waves hide HBM latency (no software prefetch, no LDS, no
//     barrier);
//   * the segment maximum M is reduced first (DPP), so every lane accumulates
//     against the exact M with no rescaling: one fma, one v_exp_f32, one add
//     and one fma per element;
//   * z and s2 are summed in a fixed DPP tree;
//   * the combine kernel folds the segments of a row, one wave per row, in a
//     fixed order.
// No device-scope fence is used anywhere (on this multi-XCD part a
// device-scope release writes back the XCD's L2); the combine runs as a
// second, small kernel.
//
// Logits that are not finite (or a segment whose maximum is not) make the
// fast statistics NaN; such a segment is recomputed by an exact
// element-by-element path that gives -inf entries weight 0, makes rows with
// NaN or +inf entries NaN, and keeps the argmax rule (lowest index, NaN
// ignored).
#include <math.h>

#include <type_traits>

#include "ec_device.h"
#include "ec_launch.h"
#include "ec_softmax_stats.h"

namespace ec {

namespace {

constexpr int32_t kRedo = -1;     // partial marker: the combine recomputes this segment exactly

template <typename T> struct VecOf;
template <> struct VecOf<float> { typedef f32x4 type; };
template <> struct VecOf<bf16_t> { typedef u32x4 type; };

constexpr int kVPT = 8;   // 16-byte vectors per lane in a full segment

constexpr int64_t seg_elems(int per_vec) { return int64_t(kVPT) * kWave * per_vec; }

// Maximum of the elements of one fp32 vector, NaN-propagating (IEEE 754-2019
// maximum, v_maximum3_f32: no input canonicalisation, two elements per
// instruction); a NaN maximum sends the segment to the exact path.
__device__ __forceinline__ float max2(float a, float b) { return __builtin_elementwise_maximum(a, b); }
__device__ __forceinline__ float vec_max(const f32x4& v) {
  return max2(max2(v.x, v.y), max2(v.z, v.w));
}

// Packed maximum of bf16 pairs using the fp16 NaN-propagating maximum
// (v_pk_maximum3_f16).  Read as fp16, a bf16 bit pattern orders the same way
// for every value below 2^121 in magnitude (both formats are sign-magnitude
// with the exponent in the high bits); bf16 infinities, NaNs and values of
// 2^121 or more read as fp16 NaNs, which the maximum propagates, and such a
// segment then fails the finiteness check and takes the exact path.
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pk_max3(uint32_t a, uint32_t b, uint32_t c) {
  const f16x2 x = __builtin_bit_cast(f16x2, a), y = __builtin_bit_cast(f16x2, b);
  const f16x2 z = __builtin_bit_cast(f16x2, c);
  return __builtin_bit_cast(uint32_t, __builtin_elementwise_maximum(__builtin_elementwise_maximum(x, y), z));
}
constexpr uint32_t kPkNegInf = 0xfc00fc00u;   // fp16 -inf in both halves (padding)

__device__ __forceinline__ EntropyPartial redo_partial() {
  EntropyPartial p;
  p.m = NAN; p.z = NAN; p.s2 = NAN; p.idx = kRedo;
  return p;
}

// Butterfly merge over the 64 lanes; the lower lane's run always goes first,
// so every lane ends with the same, order-fixed result.
__device__ __forceinline__ EntropyPartial wave_merge(EntropyPartial mine, int lane) {
#pragma unroll
  for (int o = 1; o < kWave; o <<= 1) {
    EntropyPartial other;
    other.m = __shfl_xor(mine.m, o, kWave);
    other.z = __shfl_xor(mine.z, o, kWave);
    other.s2 = __shfl_xor(mine.s2, o, kWave);
    other.idx = __shfl_xor(mine.idx, o, kWave);
    mine = (lane & o) ? merge(other, mine) : merge(mine, other);
  }
  return mine;
}

// Exact element-by-element statistics of one segment, any values.
template <typename T>
__device__ EntropyPartial exact_segment(const T* __restrict__ rp, int64_t e0, int64_t e1,
                                        int64_t nvec, int lane) {
  constexpr int E = Elem<T>::kPerVec;
  SafeAcc acc;
  for (int64_t k = lane; k < nvec; k += kWave) {
    const int64_t base = e0 + k * E;
#pragma unroll
    for (int j = 0; j < E; ++j) acc.add(Elem<T>::load(rp, base + j), int32_t(base + j));
  }
  if (lane == 0)
    for (int64_t j = e0 + nvec * E; j < e1; ++j) acc.add(Elem<T>::load(rp, j), int32_t(j));
  return wave_merge(acc.result(), lane);
}

// One wave per (row, segment) unit; segments are kVPT * 64 vectors long.  All
// loads of the unit are issued first (indices clamped into the segment, so the
// loads are unconditional), then the wave reduces the segment maximum with
// DPP, sums 2^u and 2^u u against it, and lane 0 writes the partial.  No LDS
// and no barrier: HBM latency is hidden by the other resident waves.  A
// segment whose fast statistics are not finite (or that holds only a few
// trailing elements) is marked kRedo and recomputed exactly by the combine
// kernel, which keeps that rare code out of this kernel's register budget.
template <typename T>
__global__ __launch_bounds__(256) void entropy_partials_kernel(
    const T* __restrict__ logits, int64_t stride, int64_t V, int64_t n_rows,
    const int32_t* __restrict__ n_rows_dev, int P, EntropyPartial* __restrict__ part) {
  using Vec = typename VecOf<T>::type;
  constexpr int E = Elem<T>::kPerVec;
  const int lane = threadIdx.x & (kWave - 1);
  // readfirstlane: the wave index is uniform, so the segment geometry and the
  // base address live in scalar registers and the loads take 32-bit offsets
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int64_t u = int64_t(blockIdx.x) * (256 / kWave) + wave;
  int64_t nr = n_rows;
  if (n_rows_dev != nullptr) nr = min(nr, int64_t(max(0, *n_rows_dev)));
  if (u >= nr * P) return;                                   // wave-uniform
  const int64_t row = u / P;
  const int64_t e0 = (u - row * P) * seg_elems(E);
  const int64_t e1 = min(V, e0 + seg_elems(E));
  const int nvec = int((e1 - e0) / E);
  const T* rp = logits + row * stride;
  if (nvec == 0) {                                           // fewer than E elements
    if (lane == 0) part[u] = redo_partial();
    return;
  }
  // uniform base + 32-bit unsigned per-lane byte offset: scalar-base loads
  const char* base = reinterpret_cast<const char*>(rp + e0);
  Vec d[kVPT];
#pragma unroll
  for (int j = 0; j < kVPT; ++j) {
    const uint32_t off = uint32_t(min(lane + j * kWave, nvec - 1)) * uint32_t(sizeof(Vec));
    d[j] = *reinterpret_cast<const Vec*>(base + off);
  }
  const bool full = (nvec == kVPT * kWave);
  const int64_t tail0 = e0 + int64_t(nvec) * E;              // < E trailing elements: lane 0
  const bool has_tail = (lane == 0) && (tail0 < e1);

  // ---- segment maximum (per vector kept for the argmax)
  constexpr bool kBf16 = std::is_same<T, bf16_t>::value;
  float vm[kVPT];           // fp32: per-vector maximum
  uint32_t vp[kVPT];        // bf16: per-vector packed maximum (even / odd elements)
  float tm;
  if constexpr (kBf16) {
#pragma unroll
    for (int j = 0; j < kVPT; ++j) {
      const uint32_t* w = reinterpret_cast<const uint32_t*>(&d[j]);
      vp[j] = pk_max3(pk_max3(w[0], w[1], w[2]), w[3], w[3]);
      if (!full && lane + j * kWave >= nvec) vp[j] = kPkNegInf;
    }
    uint32_t t = vp[0];
#pragma unroll
    for (int j = 1; j + 1 < kVPT; j += 2) t = pk_max3(t, vp[j], vp[j + 1]);
    if constexpr ((kVPT & 1) == 0) t = pk_max3(t, vp[kVPT - 1], vp[kVPT - 1]);
    // both halves padding: -inf, not the bf16 value 0xfc00
    const float lo = ((t & 0xffffu) == 0xfc00u) ? -INFINITY : bf16_lo(t);
    const float hi = ((t >> 16) == 0xfc00u) ? -INFINITY : bf16_hi(t);
    tm = max2(lo, hi);
  } else {
#pragma unroll
    for (int j = 0; j < kVPT; ++j) {
      vm[j] = vec_max(d[j]);
      if (!full && lane + j * kWave >= nvec) vm[j] = -INFINITY;
    }
    tm = vm[0];
#pragma unroll
    for (int j = 1; j < kVPT; ++j) tm = max2(tm, vm[j]);
  }
  if (has_tail)
    for (int64_t j = tail0; j < e1; ++j) tm = max2(tm, Elem<T>::load(rp, j));
  const float M = wave_max_dpp(tm);

  // ---- sums against the exact segment maximum
  const float mL = M * kLog2e;
  float z0 = 0.f, z1 = 0.f, s0 = 0.f, s1 = 0.f;
  if (full) {
#pragma unroll
    for (int j = 0; j < kVPT; ++j) {
      float x[E];
      unpack16(d[j], x);
#pragma unroll
      for (int k = 0; k < E; k += 2) {
        const float u0 = fmaf(x[k], kLog2e, -mL);
        const float u1 = fmaf(x[k + 1], kLog2e, -mL);
        const float q0 = fast_exp2(u0);
        const float q1 = fast_exp2(u1);
        z0 += q0;
        z1 += q1;
        s0 = fmaf(q0, u0, s0);
        s1 = fmaf(q1, u1, s1);
      }
    }
  } else {                                                   // last segment of a row
#pragma unroll
    for (int j = 0; j < kVPT; ++j) {
      const bool ok = lane + j * kWave < nvec;
      float x[E];
      unpack16(d[j], x);
#pragma unroll
      for (int k = 0; k < E; k += 2) {
        const float u0 = ok ? fmaf(x[k], kLog2e, -mL) : 0.f;
        const float u1 = ok ? fmaf(x[k + 1], kLog2e, -mL) : 0.f;
        const float q0 = ok ? fast_exp2(u0) : 0.f;
        const float q1 = ok ? fast_exp2(u1) : 0.f;
        z0 += q0;
        z1 += q1;
        s0 = fmaf(q0, u0, s0);
        s1 = fmaf(q1, u1, s1);
      }
    }
  }
  if (has_tail)
    for (int64_t j = tail0; j < e1; ++j) {
      const float u0 = fmaf(Elem<T>::load(rp, j), kLog2e, -mL);
      const float q0 = fast_exp2(u0);
      z0 += q0;
      s0 = fmaf(q0, u0, s0);
    }

  // ---- argmax: the lowest index holding M; only the lane(s) whose vectors
  // reach M scan, and only the first such vector
  int idx = kNoIdx;
  if (tm == M) {
#pragma unroll
    for (int j = 0; j < kVPT; ++j) {
      bool has;
      if constexpr (kBf16) has = (bf16_lo(vp[j]) == M) || (bf16_hi(vp[j]) == M);
      else has = (vm[j] == M);
      if (idx == kNoIdx && has) {
        float x[E];
        unpack16(d[j], x);
        int k0 = E;
#pragma unroll
        for (int k = E - 1; k >= 0; --k) k0 = (x[k] == M) ? k : k0;
        idx = int32_t(e0 + int64_t(lane + j * kWave) * E + k0);
      }
    }
    if (idx == kNoIdx && has_tail)
      for (int64_t j = tail0; j < e1; ++j)
        if (Elem<T>::load(rp, j) == M) { idx = int32_t(j); break; }
  }
  const float Z = wave_sum_dpp(z0 + z1);
  const float S = wave_sum_dpp(s0 + s1);
  const int I = wave_min_i_dpp(idx);
  const bool ok = (Z > 0.f) && (Z < INFINITY) && (fabsf(S) < INFINITY) && (fabsf(M) < INFINITY);
  EntropyPartial p = redo_partial();
  if (ok) { p.m = M; p.z = Z; p.s2 = S; p.idx = I; }
  if (lane == 0) part[u] = p;
}

// Fold the segments of each row in order, then (optionally) take E over D and
// decide.
constexpr int kCombineThreads = 1024;

// Row statistics from the merged partial.
__device__ __forceinline__ void finish_row(const EntropyPartial& acc, int64_t row,
                                           float* __restrict__ H, int32_t* __restrict__ A,
                                           float* __restrict__ p1) {
  const float z = acc.z;
  const bool ok = (z > 0.f) && (z < INFINITY);            // false for NaN
  H[row] = ok ? kLn2 * (log2f(z) - acc.s2 / z) : NAN;
  if (p1 != nullptr) p1[row] = ok ? 1.f / z : NAN;
  if (A != nullptr) A[row] = (acc.idx == kNoIdx) ? 0 : acc.idx;
}

// One wave per row: lane l folds segments l, l + 64, ... in order, then the
// lanes merge in a fixed butterfly.  Segments marked kRedo are first replaced
// by their exact statistics, computed by the whole wave.  Every lane returns
// the row's merged statistics.
template <typename T>
__device__ __forceinline__ EntropyPartial combine_row(const T* __restrict__ logits, int64_t stride,
                                                      int64_t V,
                                                      const EntropyPartial* __restrict__ part,
                                                      int P, int64_t row, int lane) {
  constexpr int E = Elem<T>::kPerVec;
  const T* rp = logits + row * stride;
  EntropyPartial acc = empty_partial();
  for (int b = 0; b < P; b += kWave) {                    // wave-uniform loop
    const int s = b + lane;
    EntropyPartial p = (s < P) ? part[row * P + s] : empty_partial();
    uint64_t redo = __ballot(s < P && p.idx == kRedo);
    while (redo != 0) {
      const int l = __ffsll(static_cast<unsigned long long>(redo)) - 1;
      redo &= redo - 1;
      const int64_t e0 = int64_t(b + l) * seg_elems(E);
      const int64_t e1 = min(V, e0 + seg_elems(E));
      const EntropyPartial q = exact_segment<T>(rp, e0, e1, (e1 - e0) / E, lane);
      if (lane == l) p = q;
    }
    acc = merge(acc, p);
  }
  return wave_merge(acc, lane);
}

template <typename T>
__global__ __launch_bounds__(256) void entropy_combine_kernel(
    const T* __restrict__ logits, int64_t stride, int64_t V,
    const EntropyPartial* __restrict__ part, int64_t n_rows, const int32_t* __restrict__ n_rows_dev,
    int P, float* __restrict__ H, int32_t* __restrict__ A, float* __restrict__ p1) {
  const int lane = threadIdx.x & (kWave - 1);
  const int64_t row = int64_t(blockIdx.x) * (256 / kWave) + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  int64_t nr = n_rows;
  if (n_rows_dev != nullptr) nr = min(nr, int64_t(max(0, *n_rows_dev)));
  if (row >= nr) return;                                  // wave-uniform
  const EntropyPartial acc = combine_row<T>(logits, stride, V, part, P, row, lane);
  if (lane == 0) finish_row(acc, row, H, A, p1);
}

__global__ __launch_bounds__(kCombineThreads) void entropy_decide_kernel(
    int64_t n_rows, const float* __restrict__ H, const int32_t* __restrict__ D,
    const int32_t* __restrict__ nD, int32_t maxD, float tau, float* __restrict__ e_max,
    int32_t* __restrict__ flag) {
  const int tid = threadIdx.x;
  int64_t count = n_rows;
  if (D != nullptr) count = min(int64_t(max(0, *nD)), int64_t(maxD));
  float best = -INFINITY;
  int nan = 0;
  for (int64_t i = tid; i < count; i += kCombineThreads) {
    const float h = H[D != nullptr ? D[i] : i];
    if (h != h) nan = 1; else best = fmaxf(best, h);
  }
  best = wave_max(best);
  nan = wave_sum_i(nan);
  __shared__ float sb[kCombineThreads / kWave];
  __shared__ int sn[kCombineThreads / kWave];
  if ((tid & (kWave - 1)) == 0) { sb[tid / kWave] = best; sn[tid / kWave] = nan; }
  __syncthreads();
  if (tid == 0) {
    float b = -INFINITY;
    int n = 0;
    for (int k = 0; k < kCombineThreads / kWave; ++k) { b = fmaxf(b, sb[k]); n += sn[k]; }
    const float E = n ? NAN : b;
    *e_max = E;
    *flag = (n || E > tau) ? 1 : 0;
  }
}

// ---- the step's decode and decision, in one workgroup
//
// The few logit rows of a step (the block's candidates, or the rows a caller
// decoded) are folded here, one wave per row as in entropy_combine_kernel,
// and the decision follows in the same workgroup:
//  * choose (cand_pos != nullptr): the n_unmask candidates of largest p1 are
//    unmasked (ties to the lower position, NaN last), decode to their argmax
//    and join the history in ascending position order; E = max H over them;
//  * decide-all (cand_pos == nullptr): E = max H over every row.
// Then flag = (E > tau) || isnan(E) (-inf when nothing was decoded).
// EntropyCache, Chinese summary page §2.2 (decode, E_{t+1}, threshold rule)
// and Portuguese page §2 (decode history).  The pages do not fix the decode
// rule; the ranking by top-1 probability is this library's reading.
constexpr int kStepThreads = 1024;

__device__ __forceinline__ bool better(float pj, int posj, float pi, int posi) {
  const bool nj = (pj != pj), ni = (pi != pi);
  if (nj != ni) return ni;                 // a number beats NaN
  if (!nj && pj != pi) return pj > pi;
  return posj < posi;                      // equal (or both NaN): lower position first
}

// Partials written by the LM head's epilogue (one per row and tile group, no
// segment to redo): 32 lanes per row, lane q folding partials q, q + 32, ...
// in order, all of a batch's loads issued first (24 per lane: one batch up to
// 768 partials per row), then a butterfly over the 32 lanes (lower lane
// first).  Every lane of the row returns its statistics.
constexpr int kFoldBatch = 24;
__device__ __forceinline__ EntropyPartial fold_row32(const EntropyPartial* __restrict__ part, int P,
                                                     int row, int q) {
  const EntropyPartial* rp = part + int64_t(row) * P;
  EntropyPartial acc = empty_partial();
  for (int b = 0; b < P; b += 32 * kFoldBatch) {          // uniform across the row's lanes
    EntropyPartial v[kFoldBatch];
#pragma unroll
    for (int i = 0; i < kFoldBatch; ++i) {
      const int k = b + 32 * i + q;
      v[i] = (k < P) ? rp[k] : empty_partial();
    }
#pragma unroll
    for (int i = 0; i < kFoldBatch; ++i) acc = merge(acc, v[i]);
  }
#pragma unroll
  for (int o = 1; o < 32; o <<= 1) {
    EntropyPartial other;
    other.m = __shfl_xor(acc.m, o, 32);
    other.z = __shfl_xor(acc.z, o, 32);
    other.s2 = __shfl_xor(acc.s2, o, 32);
    other.idx = __shfl_xor(acc.idx, o, 32);
    acc = (q & o) ? merge(other, acc) : merge(acc, other);
  }
  return acc;
}

// FUSED: the rows' partials come from the LM head (at most 32 rows, P per
// row, see fold_row32) and logits is not read; otherwise from
// entropy_partials_kernel (P segments per row, folded by combine_row).
template <typename T, bool FUSED = false>
__global__ __launch_bounds__(kStepThreads) void entropy_step_kernel(
    const T* __restrict__ logits, int64_t stride, int64_t V,
    const EntropyPartial* __restrict__ part, int P, int32_t max_rows,
    const int32_t* __restrict__ n_rows_dev, float* __restrict__ H, int32_t* __restrict__ A,
    float* __restrict__ p1, const int32_t* __restrict__ cand_pos, int32_t n_unmask, float tau,
    int32_t* __restrict__ chosen, int32_t* __restrict__ n_chosen, int32_t* __restrict__ tokens,
    uint8_t* __restrict__ is_masked, int32_t* __restrict__ history,
    int32_t* __restrict__ history_len, int32_t history_cap, float* __restrict__ e_max,
    int32_t* __restrict__ flag) {
  __shared__ float s_h[kStepThreads];
  __shared__ float s_p1[kStepThreads];
  __shared__ int s_am[kStepThreads];
  __shared__ int s_pos[kStepThreads];
  __shared__ int s_cnt[kStepThreads / kWave + 1];
  __shared__ float s_max[kStepThreads / kWave];
  __shared__ int s_nan[kStepThreads / kWave];
  constexpr int kWaves = kStepThreads / kWave;
  const int tid = threadIdx.x, lane = tid & (kWave - 1);
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const bool choose = (cand_pos != nullptr);
  const int nc = n_rows_dev != nullptr ? min(max(0, *n_rows_dev), max_rows) : max_rows;
  // every per-candidate load goes out at once (the arrays hold max_rows entries)
  const int posi = (choose && tid < max_rows) ? cand_pos[tid] : 0;
  const int hl = choose ? *history_len : 0;
  if constexpr (FUSED) {
    const int row = tid >> 5, q = tid & 31;
    if (row < nc) {                                        // uniform across the row's 32 lanes
      const EntropyPartial acc = fold_row32(part, P, row, q);
      if (q == 0) {
        finish_row(acc, row, H, A, p1);
        finish_row(acc, row, s_h, s_am, s_p1);
      }
    }
  } else {
    for (int row = w; row < nc; row += kWaves) {           // wave-uniform
      const EntropyPartial acc = combine_row<T>(logits, stride, V, part, P, row, lane);
      if (lane == 0) {
        finish_row(acc, row, H, A, p1);
        finish_row(acc, row, s_h, s_am, s_p1);
      }
    }
  }
  if (tid < nc) s_pos[tid] = posi;
  __syncthreads();
  float hmax = -INFINITY;
  int hnan = 0;
  int total = nc;
  if (choose) {
    const int ns = min(n_unmask, nc);
    bool pick = false;
    float pi = 0.f;
    if (tid < nc) {
      pi = s_p1[tid];
      int rank = 0;
      for (int j = 0; j < nc; ++j) rank += better(s_p1[j], s_pos[j], pi, posi) ? 1 : 0;
      pick = rank < ns;
    }
    // ascending-position slot of each chosen candidate (candidates are ascending)
    const int v = pick ? 1 : 0;
    int incl = v;
#pragma unroll
    for (int o = 1; o < kWave; o <<= 1) {
      const int t = __shfl_up(incl, o, kWave);
      if (lane >= o) incl += t;
    }
    if (lane == kWave - 1) s_cnt[w] = incl;
    __syncthreads();
    if (tid == 0) {
      int acc = 0;
      for (int k = 0; k < kWaves; ++k) { const int t = s_cnt[k]; s_cnt[k] = acc; acc += t; }
      s_cnt[kWaves] = acc;
    }
    __syncthreads();
    total = s_cnt[kWaves];
    if (pick) {
      const int slot = s_cnt[w] + incl - v;
      chosen[slot] = posi;
      tokens[posi] = s_am[tid];
      is_masked[posi] = 0;
      // Slots that differ by history_cap share a ring entry; only the newest
      // history_cap of this step's slots are written, so each entry has one writer.
      if (slot >= total - history_cap) history[(hl + slot) % history_cap] = posi;
      const float h = s_h[tid];
      if (h != h) hnan = 1; else hmax = h;
    }
  } else if (tid < nc) {
    const float h = s_h[tid];
    if (h != h) hnan = 1; else hmax = h;
  }
  hmax = wave_max(hmax);
  hnan = wave_sum_i(hnan);
  if (lane == 0) { s_max[w] = hmax; s_nan[w] = hnan; }
  __syncthreads();
  if (tid == 0) {
    float b = -INFINITY;
    int n = 0;
    for (int k = 0; k < kWaves; ++k) { b = fmaxf(b, s_max[k]); n += s_nan[k]; }
    const float E = n ? NAN : b;
    if (choose) {
      *n_chosen = total;
      *history_len = hl + total;
    }
    *e_max = E;
    *flag = (n || E > tau) ? 1 : 0;
  }
}

}  // namespace

static_assert(kStepThreads == kStepMaxRows, "one thread per candidate row");
int32_t step_max_rows() { return kStepThreads; }

hipError_t launch_entropy_step(const void* logits, int dtype, int32_t max_rows,
                               const int32_t* n_rows_dev, int64_t V, int64_t stride, float* H,
                               int32_t* argmax, float* p1, const int32_t* cand_pos,
                               int32_t n_unmask, float tau, int32_t* chosen, int32_t* n_chosen,
                               int32_t* tokens, uint8_t* is_masked, int32_t* history,
                               int32_t* history_len, int32_t history_cap, float* e_max,
                               int32_t* flag, void* ws, hipStream_t s) {
  if (max_rows < 1 || max_rows > kStepThreads) return hipErrorInvalidValue;
  const int P = entropy_segments(V, dtype);
  EntropyPartial* part = static_cast<EntropyPartial*>(ws);
  constexpr int kUnitsPerWG = 256 / kWave;
  const unsigned grid = unsigned((int64_t(max_rows) * P + kUnitsPerWG - 1) / kUnitsPerWG);
  constexpr size_t kResidencyLds = 32 * 1024;            // as in launch_entropy
  if (dtype == 1) {
    hipLaunchKernelGGL(entropy_partials_kernel<bf16_t>, dim3(grid), dim3(256), kResidencyLds, s,
                       static_cast<const bf16_t*>(logits), stride, V, int64_t(max_rows), n_rows_dev,
                       P, part);
  } else {
    hipLaunchKernelGGL(entropy_partials_kernel<float>, dim3(grid), dim3(256), kResidencyLds, s,
                       static_cast<const float*>(logits), stride, V, int64_t(max_rows), n_rows_dev,
                       P, part);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (dtype == 1)
    hipLaunchKernelGGL(entropy_step_kernel<bf16_t>, dim3(1), dim3(kStepThreads), 0, s,
                       static_cast<const bf16_t*>(logits), stride, V, part, P, max_rows, n_rows_dev,
                       H, argmax, p1, cand_pos, n_unmask, tau, chosen, n_chosen, tokens, is_masked,
                       history, history_len, history_cap, e_max, flag);
  else
    hipLaunchKernelGGL(entropy_step_kernel<float>, dim3(1), dim3(kStepThreads), 0, s,
                       static_cast<const float*>(logits), stride, V, part, P, max_rows, n_rows_dev,
                       H, argmax, p1, cand_pos, n_unmask, tau, chosen, n_chosen, tokens, is_masked,
                       history, history_len, history_cap, e_max, flag);
  return hipGetLastError();
}

hipError_t launch_entropy_step_fused(const EntropyPartial* part, int32_t P, int32_t max_rows,
                                     const int32_t* n_rows_dev, float* H, int32_t* argmax, float* p1,
                                     const int32_t* cand_pos, int32_t n_unmask, float tau,
                                     int32_t* chosen, int32_t* n_chosen, int32_t* tokens,
                                     uint8_t* is_masked, int32_t* history, int32_t* history_len,
                                     int32_t history_cap, float* e_max, int32_t* flag, hipStream_t s) {
  if (max_rows < 1 || max_rows > kLmStatRows || P < 1) return hipErrorInvalidValue;
  hipLaunchKernelGGL((entropy_step_kernel<bf16_t, true>), dim3(1), dim3(kStepThreads), 0, s,
                     static_cast<const bf16_t*>(nullptr), int64_t(0), int64_t(0), part, int(P), max_rows,
                     n_rows_dev, H, argmax, p1, cand_pos, n_unmask, tau, chosen, n_chosen, tokens,
                     is_masked, history, history_len, history_cap, e_max, flag);
  return hipGetLastError();
}

int device_cu_count() {
  static int cached = 0;
  if (cached == 0) {
    int dev = 0, n = 0;
    if (hipGetDevice(&dev) == hipSuccess &&
        hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && n > 0)
      cached = n;
    else
      cached = 256;
  }
  return cached;
}

int entropy_segments(int64_t V, int dtype) {
  const int64_t seg = seg_elems(dtype == 1 ? 8 : 4);
  return int((V + seg - 1) / seg);
}

size_t entropy_ws_bytes(int64_t n_rows, int64_t V, int dtype) {
  return size_t(n_rows) * size_t(entropy_segments(V, dtype)) * sizeof(EntropyPartial);
}

hipError_t launch_entropy(const void* logits, int dtype, int64_t n_rows, const int32_t* n_rows_dev,
                          int64_t V, int64_t stride, float* H, int32_t* argmax, float* p1,
                          const int32_t* D, const int32_t* nD, int32_t maxD, float tau,
                          float* e_max, int32_t* flag, void* ws, hipStream_t s) {
  const int P = entropy_segments(V, dtype);
  EntropyPartial* part = static_cast<EntropyPartial*>(ws);
  constexpr int kUnitsPerWG = 256 / kWave;
  const int64_t units = n_rows * P;
  const unsigned grid = unsigned((units + kUnitsPerWG - 1) / kUnitsPerWG);
  // The kernel uses no LDS; the launch reserves 32 KiB per workgroup anyway,
  // which caps residency at five workgroups (20 waves) per CU.  More resident
  // waves keep more reads in flight but lower the HBM efficiency of this
  // stream (measured: 8 per CU 182 us, 5 per CU 170 us for 4096 x 126464 bf16).
  constexpr size_t kResidencyLds = 32 * 1024;
  if (dtype == 1)
    hipLaunchKernelGGL(entropy_partials_kernel<bf16_t>, dim3(grid), dim3(256), kResidencyLds, s,
                       static_cast<const bf16_t*>(logits), stride, V, n_rows, n_rows_dev, P, part);
  else
    hipLaunchKernelGGL(entropy_partials_kernel<float>, dim3(grid), dim3(256), kResidencyLds, s,
                       static_cast<const float*>(logits), stride, V, n_rows, n_rows_dev, P, part);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const dim3 cgrid(unsigned((n_rows + kUnitsPerWG - 1) / kUnitsPerWG));
  if (dtype == 1)
    hipLaunchKernelGGL(entropy_combine_kernel<bf16_t>, cgrid, dim3(256), 0, s,
                       static_cast<const bf16_t*>(logits), stride, V, part, n_rows, n_rows_dev, P,
                       H, argmax, p1);
  else
    hipLaunchKernelGGL(entropy_combine_kernel<float>, cgrid, dim3(256), 0, s,
                       static_cast<const float*>(logits), stride, V, part, n_rows, n_rows_dev, P,
                       H, argmax, p1);
  e = hipGetLastError();
  if (e != hipSuccess || e_max == nullptr) return e;
  hipLaunchKernelGGL(entropy_decide_kernel, dim3(1), dim3(kCombineThreads), 0, s, n_rows, H, D,
                     nD, maxD, tau, e_max, flag);
  return hipGetLastError();
}

}  // namespace ec
