// KV drift of a full recompute (a diagnostic the step can report): 1 - cos
// between each position's stale and recomputed Value vector, concatenated over
// the KV heads, reduced per layer to the mean and the maximum over positions.
//
// EntropyCache, Chinese summary page §2.1 (first observation) and Portuguese
// page §2: the entropy of a newly decoded token tracks how far the KV cache
// drifts, measured on the Value vectors as a cosine distance.  The pages give
// no aggregation; here positions whose stale or fresh vector is all zero
// (never computed) are left out, and the mean and maximum are taken over the
// rest (NaN when none is left).
//
// Every kernel reads the step's mode flag and exits at once on a partial step,
// so a step's launch sequence never depends on the decision.
#include <math.h>

#include "ec_device.h"
#include "ec_launch.h"

namespace ec {

namespace {

// Copy columns [0, L8) of the nrow rows of a transposed Value cache [nrow, L_cap]
// in 16-byte vectors (L8: L rounded up to a whole vector, <= L_cap).
template <typename T>
__global__ __launch_bounds__(256) void vsnap_kernel(const int32_t* __restrict__ flag,
                                                   const T* __restrict__ vc, T* __restrict__ snap,
                                                   int nrow, int L8, int L_cap) {
  if (*flag == 0) return;
  constexpr int E = Elem<T>::kPerVec;
  const int64_t per_row = L8 / E;
  const int64_t total = int64_t(nrow) * per_row;
  for (int64_t i = int64_t(blockIdx.x) * 256 + threadIdx.x; i < total; i += int64_t(gridDim.x) * 256) {
    const int64_t r = i / per_row, c = i - r * per_row;
    const int64_t off = r * L_cap + c * E;
    *reinterpret_cast<u32x4*>(snap + off) = *reinterpret_cast<const u32x4*>(vc + off);
  }
}

// Per-position 1 - cos(stale, fresh): a workgroup owns 64 consecutive positions
// (one per lane, so every load is a coalesced row segment) and its 16 waves
// split the nrow rows; the waves' sums are added in a fixed order.
constexpr int kDriftWaves = 16;

template <typename T>
__global__ __launch_bounds__(kDriftWaves * 64) void vdrift_kernel(
    const int32_t* __restrict__ flag, const T* __restrict__ snap, const T* __restrict__ vc, int nrow,
    int L, int L_cap, float* __restrict__ dpos) {
  if (*flag == 0) return;
  __shared__ float part[kDriftWaves][3][64];
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int p = blockIdx.x * 64 + lane;
  float dot = 0.f, na = 0.f, nb = 0.f;
  if (p < L)
    for (int r = w; r < nrow; r += kDriftWaves) {
      const float a = Elem<T>::load(snap, int64_t(r) * L_cap + p);
      const float b = Elem<T>::load(vc, int64_t(r) * L_cap + p);
      dot = fmaf(a, b, dot);
      na = fmaf(a, a, na);
      nb = fmaf(b, b, nb);
    }
  part[w][0][lane] = dot;
  part[w][1][lane] = na;
  part[w][2][lane] = nb;
  __syncthreads();
  if (w == 0 && p < L) {
    float s0 = 0.f, s1 = 0.f, s2 = 0.f;
    for (int k = 0; k < kDriftWaves; ++k) {
      s0 += part[k][0][lane];
      s1 += part[k][1][lane];
      s2 += part[k][2][lane];
    }
    dpos[p] = (s1 > 0.f && s2 > 0.f) ? 1.f - s0 / sqrtf(s1 * s2) : NAN;
  }
}

// Mean and maximum of the per-position distances that are not NaN.
constexpr int kFinishThreads = 1024;

__global__ __launch_bounds__(kFinishThreads) void vdrift_finish_kernel(
    const int32_t* __restrict__ flag, const float* __restrict__ dpos, int L, float* __restrict__ out) {
  if (*flag == 0) return;
  const int tid = threadIdx.x;
  float sum = 0.f, mx = -INFINITY;
  int cnt = 0;
  for (int p = tid; p < L; p += kFinishThreads) {
    const float d = dpos[p];
    if (d == d) { sum += d; mx = fmaxf(mx, d); ++cnt; }
  }
  sum = wave_sum(sum);
  mx = wave_max(mx);
  cnt = wave_sum_i(cnt);
  __shared__ float ss[kFinishThreads / 64], sm[kFinishThreads / 64];
  __shared__ int sc[kFinishThreads / 64];
  if ((tid & 63) == 0) { ss[tid / 64] = sum; sm[tid / 64] = mx; sc[tid / 64] = cnt; }
  __syncthreads();
  if (tid == 0) {
    float s = 0.f, m = -INFINITY;
    int c = 0;
    for (int k = 0; k < kFinishThreads / 64; ++k) { s += ss[k]; m = fmaxf(m, sm[k]); c += sc[k]; }
    out[0] = c ? s / float(c) : NAN;
    out[1] = c ? m : NAN;
  }
}

}  // namespace

size_t value_drift_ws_bytes(int dtype, int nrow, int L_cap) {
  const size_t es = dtype == 1 ? 2 : 4;
  return size_t(nrow) * size_t(L_cap) * es + size_t(L_cap) * sizeof(float);
}

hipError_t launch_value_drift_snapshot(int dtype, const int32_t* flag, const void* v_cache, int nrow,
                                       int L, int L_cap, void* ws, hipStream_t s) {
  const int E = dtype == 1 ? 8 : 4;
  const int L8 = (L + E - 1) / E * E;          // <= L_cap: rows are whole 16-byte vectors
  const int64_t total = int64_t(nrow) * (L8 / E);
  int64_t blocks = (total + 255) / 256;
  const int64_t cap = 4 * int64_t(device_cu_count());
  if (blocks > cap) blocks = cap;
  if (blocks < 1) blocks = 1;
  const unsigned grid = unsigned(blocks);
  if (dtype == 1)
    hipLaunchKernelGGL(vsnap_kernel<bf16_t>, dim3(grid), dim3(256), 0, s, flag,
                       static_cast<const bf16_t*>(v_cache), static_cast<bf16_t*>(ws), nrow, L8, L_cap);
  else
    hipLaunchKernelGGL(vsnap_kernel<float>, dim3(grid), dim3(256), 0, s, flag,
                       static_cast<const float*>(v_cache), static_cast<float*>(ws), nrow, L8, L_cap);
  return hipGetLastError();
}

hipError_t launch_value_drift(int dtype, const int32_t* flag, const void* v_cache, int nrow, int L,
                              int L_cap, void* ws, float* out, hipStream_t s) {
  const size_t es = dtype == 1 ? 2 : 4;
  float* dpos = reinterpret_cast<float*>(static_cast<char*>(ws) + size_t(nrow) * size_t(L_cap) * es);
  const dim3 grid(unsigned((L + 63) / 64));
  if (dtype == 1)
    hipLaunchKernelGGL(vdrift_kernel<bf16_t>, grid, dim3(kDriftWaves * 64), 0, s, flag,
                       static_cast<const bf16_t*>(ws), static_cast<const bf16_t*>(v_cache), nrow, L,
                       L_cap, dpos);
  else
    hipLaunchKernelGGL(vdrift_kernel<float>, grid, dim3(kDriftWaves * 64), 0, s, flag,
                       static_cast<const float*>(ws), static_cast<const float*>(v_cache), nrow, L,
                       L_cap, dpos);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(vdrift_finish_kernel, dim3(1), dim3(kFinishThreads), 0, s, flag, dpos, L, out);
  return hipGetLastError();
}

}  // namespace ec
