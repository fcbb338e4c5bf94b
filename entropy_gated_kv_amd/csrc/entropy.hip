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
//   * a row is cut into segments of 2048 16-byte vectors (16384 bf16 or 8192
//     fp32 elements);
//   * within a segment, thread t of 256 owns the 16-byte vectors t, t+256, ...
//     (8 per thread in a full segment);
//   * the segment maximum M is reduced first (DPP within each wave, then the
//     four waves), so every thread accumulates against the exact M with no
//     rescaling: one fma, one v_exp_f32, one add and one fma per element;
//   * z and s2 are summed in a fixed DPP tree, then over the waves in order;
//   * segments of a row are folded left to right by the combine kernel.
// Kernel 1 is persistent: each workgroup walks (row, segment) units with a
// stride of the grid size and prefetches the next unit's vectors into
// registers while it reduces the current one, so HBM reads stay in flight.
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

#include "ec_device.h"
#include "ec_launch.h"

namespace ec {

namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / kWave;
constexpr int32_t kNoIdx = 0x7fffffff;

__device__ __forceinline__ EntropyPartial merge(const EntropyPartial& a, const EntropyPartial& b) {
  EntropyPartial r;
  r.m = fmaxf(a.m, b.m);
  const bool ea = (a.m == -INFINITY), eb = (b.m == -INFINITY);
  const float da = ea ? 0.f : (a.m - r.m) * kLog2e;
  const float db = eb ? 0.f : (b.m - r.m) * kLog2e;
  const float ra = ea ? 0.f : fast_exp2(da);
  const float rb = eb ? 0.f : fast_exp2(db);
  r.z = a.z * ra + b.z * rb;
  r.s2 = ra * (a.s2 + da * a.z) + rb * (b.s2 + db * b.z);
  r.idx = (a.m > b.m) ? a.idx : ((b.m > a.m) ? b.idx : min(a.idx, b.idx));
  return r;
}

// Exact per-element accumulation (any value).
struct SafeAcc {
  float m = -INFINITY, z = 0.f, s2 = 0.f, best = -INFINITY;
  int32_t idx = kNoIdx;
  bool bad = false;
  __device__ __forceinline__ void add(float x, int32_t j) {
    if (x != x) { bad = true; return; }                      // NaN: ignored by argmax
    if (x > best || idx == kNoIdx) { best = x; idx = j; }   // lowest index wins ties
    if (x == INFINITY) { bad = true; return; }
    if (x == -INFINITY) return;                              // weight exactly 0
    if (x > m) {
      if (m != -INFINITY) {
        const float d = (m - x) * kLog2e;
        const float r = fast_exp2(d);
        s2 = r * (s2 + d * z);
        z = r * z;
      }
      m = x;
    }
    const float u = (x - m) * kLog2e;
    const float e = fast_exp2(u);
    z += e;
    s2 = fmaf(e, u, s2);
  }
  __device__ __forceinline__ EntropyPartial result() const {
    EntropyPartial p;
    p.m = best;          // includes +inf, so the argmax merge sees it
    p.z = bad ? NAN : z;
    p.s2 = bad ? NAN : s2;
    p.idx = idx;
    return p;
  }
};

template <typename T> struct VecOf;
template <> struct VecOf<float> { typedef f32x4 type; };
template <> struct VecOf<bf16_t> { typedef u32x4 type; };

constexpr int kVPT = 8;   // vectors per thread in a full segment

constexpr int64_t seg_elems(int per_vec) { return int64_t(kVPT) * kThreads * per_vec; }

template <typename T>
struct Unit {
  typename VecOf<T>::type v[kVPT];
};

struct UnitGeom {
  int64_t row, e0, e1, nvec;   // nvec: full 16-byte vectors in [e0, e1)
};

template <typename T>
__device__ __forceinline__ UnitGeom geom(int64_t u, int P, int64_t V) {
  constexpr int E = Elem<T>::kPerVec;
  UnitGeom g;
  g.row = u / P;
  const int seg = int(u - g.row * P);
  g.e0 = int64_t(seg) * seg_elems(E);
  g.e1 = min(V, g.e0 + seg_elems(E));
  g.nvec = (g.e1 - g.e0) / E;
  return g;
}

template <typename T>
__device__ __forceinline__ void load_unit(const T* __restrict__ logits, int64_t stride,
                                          const UnitGeom& g, int tid, Unit<T>& d) {
  using Vec = typename VecOf<T>::type;
  const Vec* vp = reinterpret_cast<const Vec*>(logits + g.row * stride + g.e0);
#pragma unroll
  for (int j = 0; j < kVPT; ++j) {
    const int64_t i = tid + j * kThreads;
    if (i < g.nvec) d.v[j] = __builtin_nontemporal_load(vp + i);
    else d.v[j] = Vec{};
  }
}

struct Shared {
  float m[kWaves];
  float z[kWaves];
  float s[kWaves];
  int idx[kWaves];
  EntropyPartial part[kWaves];
};

template <typename T>
__device__ __forceinline__ EntropyPartial exact_unit(const T* __restrict__ logits, int64_t stride,
                                                  const UnitGeom& g, int tid, Shared& sh) {
  constexpr int E = Elem<T>::kPerVec;
  const T* rp = logits + g.row * stride;
  SafeAcc acc;
  for (int64_t k = tid; k < g.nvec; k += kThreads) {
    const int64_t base = g.e0 + k * E;
#pragma unroll
    for (int j = 0; j < E; ++j) acc.add(Elem<T>::load(rp, base + j), int32_t(base + j));
  }
  if (tid == 0)
    for (int64_t j = g.e0 + g.nvec * E; j < g.e1; ++j) acc.add(Elem<T>::load(rp, j), int32_t(j));
  EntropyPartial mine = acc.result();
  const int lane = tid & (kWave - 1);
#pragma unroll
  for (int o = 1; o < kWave; o <<= 1) {
    EntropyPartial other;
    other.m = __shfl_xor(mine.m, o, kWave);
    other.z = __shfl_xor(mine.z, o, kWave);
    other.s2 = __shfl_xor(mine.s2, o, kWave);
    other.idx = __shfl_xor(mine.idx, o, kWave);
    mine = (lane & o) ? merge(other, mine) : merge(mine, other);   // lower lane first
  }
  if (lane == 0) sh.part[tid / kWave] = mine;
  __syncthreads();
  EntropyPartial r = sh.part[0];
#pragma unroll
  for (int w = 1; w < kWaves; ++w) r = merge(r, sh.part[w]);
  __syncthreads();
  return r;
}

// Fast path for one unit whose vectors are already in registers.
template <typename T>
__device__ __forceinline__ void process_unit(const T* __restrict__ logits, int64_t stride,
                                             const UnitGeom& g, const Unit<T>& d, int tid,
                                             Shared& sh, EntropyPartial* __restrict__ out,
                                             int64_t u) {
  constexpr int E = Elem<T>::kPerVec;
  const int lane = tid & (kWave - 1), w = tid / kWave;
  const bool full = (g.nvec == int64_t(kVPT) * kThreads);
  const int64_t tail0 = g.e0 + g.nvec * E;           // scalar tail [tail0, e1): thread 0
  const T* rp = logits + g.row * stride;

  // ---- phase 1: segment maximum
  float tm = -INFINITY;
#pragma unroll
  for (int j = 0; j < kVPT; ++j) {
    if (!full && tid + j * kThreads >= g.nvec) continue;
    float x[E];
    unpack16(d.v[j], x);
#pragma unroll
    for (int k = 0; k < E; ++k) tm = fmaxf(tm, x[k]);
  }
  const bool has_tail = (tid == 0) && (tail0 < g.e1);  // < E elements past the last vector
  if (has_tail)
    for (int64_t j = tail0; j < g.e1; ++j) tm = fmaxf(tm, Elem<T>::load(rp, j));
  const float wm = wave_max_dpp(tm);
  if (lane == 0) sh.m[w] = wm;
  __syncthreads();
  float M = sh.m[0];
#pragma unroll
  for (int k = 1; k < kWaves; ++k) M = fmaxf(M, sh.m[k]);

  // ---- phase 2: sums against the exact segment maximum
  const float mL = M * kLog2e;
  float z0 = 0.f, z1 = 0.f, s0 = 0.f, s1 = 0.f;
#pragma unroll
  for (int j = 0; j < kVPT; ++j) {
    if (!full && tid + j * kThreads >= g.nvec) continue;
    float x[E];
    unpack16(d.v[j], x);
#pragma unroll
    for (int k = 0; k < E; k += 2) {
      const float u0 = fmaf(x[k], kLog2e, -mL);
      const float u1 = fmaf(x[k + 1], kLog2e, -mL);
      const float e0 = fast_exp2(u0);
      const float e1 = fast_exp2(u1);
      z0 += e0;
      z1 += e1;
      s0 = fmaf(e0, u0, s0);
      s1 = fmaf(e1, u1, s1);
    }
  }
  if (has_tail)
    for (int64_t j = tail0; j < g.e1; ++j) {
      const float u0 = fmaf(Elem<T>::load(rp, j), kLog2e, -mL);
      const float e0 = fast_exp2(u0);
      z0 += e0;
      s0 = fmaf(e0, u0, s0);
    }
  // argmax: the lowest index holding M, searched only by threads whose max is M
  int idx = kNoIdx;
  if (tm == M) {
#pragma unroll
    for (int j = 0; j < kVPT; ++j) {
      if (tid + j * kThreads < g.nvec) {
        float x[E];
        unpack16(d.v[j], x);
#pragma unroll
        for (int k = E - 1; k >= 0; --k)      // scanning down leaves the lowest match
          if (x[k] == M) idx = min(idx, int32_t(g.e0 + (int64_t(tid) + j * kThreads) * E + k));
      }
    }
    if (idx == kNoIdx && has_tail)
      for (int64_t j = tail0; j < g.e1; ++j)
        if (Elem<T>::load(rp, j) == M) { idx = int32_t(j); break; }
  }
  const float wz = wave_sum_dpp(z0 + z1);
  const float ws = wave_sum_dpp(s0 + s1);
  const int wi = wave_min_i_dpp(idx);
  if (lane == 0) { sh.z[w] = wz; sh.s[w] = ws; sh.idx[w] = wi; }
  __syncthreads();
  float Z = sh.z[0], S = sh.s[0];
  int I = sh.idx[0];
#pragma unroll
  for (int k = 1; k < kWaves; ++k) { Z += sh.z[k]; S += sh.s[k]; I = min(I, sh.idx[k]); }
  const bool ok = (Z > 0.f) && (Z < INFINITY) && (fabsf(S) < INFINITY) && (fabsf(M) < INFINITY);
  if (ok) {
    if (tid == 0) {
      EntropyPartial p;
      p.m = M; p.z = Z; p.s2 = S; p.idx = I;
      out[u] = p;
    }
  } else {                                       // uniform across the workgroup
    const EntropyPartial p = exact_unit<T>(logits, stride, g, tid, sh);
    if (tid == 0) out[u] = p;
  }
}

template <typename T>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(4, 8)))
void entropy_partials_kernel(
    const T* __restrict__ logits, int64_t stride, int64_t V, int64_t n_rows,
    const int32_t* __restrict__ n_rows_dev, int P, EntropyPartial* __restrict__ part) {
  __shared__ Shared sh;
  const int tid = threadIdx.x;
  int64_t nr = n_rows;
  if (n_rows_dev != nullptr) nr = min(nr, int64_t(max(0, *n_rows_dev)));
  const int64_t total = nr * P;
  const int64_t G = gridDim.x;
  int64_t u = blockIdx.x;
  if (u >= total) return;
  Unit<T> a, b;
  UnitGeom ga = geom<T>(u, P, V), gb = ga;
  load_unit<T>(logits, stride, ga, tid, a);
  while (true) {
    int64_t un = u + G;
    if (un < total) { gb = geom<T>(un, P, V); load_unit<T>(logits, stride, gb, tid, b); }
    process_unit<T>(logits, stride, ga, a, tid, sh, part, u);
    u = un;
    if (u >= total) break;
    un = u + G;
    if (un < total) { ga = geom<T>(un, P, V); load_unit<T>(logits, stride, ga, tid, a); }
    process_unit<T>(logits, stride, gb, b, tid, sh, part, u);
    u = un;
    if (u >= total) break;
  }
}

// Fold the segments of each row in order, then (optionally) take E over D and
// decide.
constexpr int kCombineThreads = 1024;

__device__ __forceinline__ void finish_row(const EntropyPartial* __restrict__ part, int64_t row,
                                           int P, float* __restrict__ H, int32_t* __restrict__ A,
                                           float* __restrict__ p1) {
  EntropyPartial acc = part[row * P];
  for (int s = 1; s < P; ++s) acc = merge(acc, part[row * P + s]);
  const float z = acc.z;
  const bool ok = (z > 0.f) && (z < INFINITY);            // false for NaN
  H[row] = ok ? kLn2 * (log2f(z) - acc.s2 / z) : NAN;
  if (p1 != nullptr) p1[row] = ok ? 1.f / z : NAN;
  if (A != nullptr) A[row] = (acc.idx == kNoIdx) ? 0 : acc.idx;
}

__global__ __launch_bounds__(256) void entropy_combine_kernel(
    const EntropyPartial* __restrict__ part, int64_t n_rows, const int32_t* __restrict__ n_rows_dev,
    int P, float* __restrict__ H, int32_t* __restrict__ A, float* __restrict__ p1) {
  const int64_t row = int64_t(blockIdx.x) * 256 + threadIdx.x;
  int64_t nr = n_rows;
  if (n_rows_dev != nullptr) nr = min(nr, int64_t(max(0, *n_rows_dev)));
  if (row < nr) finish_row(part, row, P, H, A, p1);
}

__global__ __launch_bounds__(kCombineThreads) void entropy_decide_kernel(
    const EntropyPartial* __restrict__ part, int64_t n_rows, int P, int do_rows,
    float* __restrict__ H, int32_t* __restrict__ A, float* __restrict__ p1,
    const int32_t* __restrict__ D, const int32_t* __restrict__ nD, int32_t maxD, float tau,
    float* __restrict__ e_max, int32_t* __restrict__ flag) {
  const int tid = threadIdx.x;
  if (do_rows)
    for (int64_t row = tid; row < n_rows; row += kCombineThreads) finish_row(part, row, P, H, A, p1);
  __syncthreads();                                        // H of every row visible to the workgroup
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

}  // namespace

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
  const int64_t units = n_rows * P;
  const int64_t cap = int64_t(device_cu_count()) * 4;
  const int64_t grid = units < cap ? units : cap;
  if (dtype == 1)
    hipLaunchKernelGGL(entropy_partials_kernel<bf16_t>, dim3(unsigned(grid)), dim3(kThreads), 0, s,
                       static_cast<const bf16_t*>(logits), stride, V, n_rows, n_rows_dev, P, part);
  else
    hipLaunchKernelGGL(entropy_partials_kernel<float>, dim3(unsigned(grid)), dim3(kThreads), 0, s,
                       static_cast<const float*>(logits), stride, V, n_rows, n_rows_dev, P, part);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  // Small standalone batches: one workgroup folds the rows and decides.
  const bool one_wg = (e_max != nullptr) && n_rows <= 16384 && n_rows_dev == nullptr;
  if (!one_wg) {
    hipLaunchKernelGGL(entropy_combine_kernel, dim3(unsigned((n_rows + 255) / 256)), dim3(256), 0, s,
                       part, n_rows, n_rows_dev, P, H, argmax, p1);
    e = hipGetLastError();
    if (e != hipSuccess || e_max == nullptr) return e;
  }
  hipLaunchKernelGGL(entropy_decide_kernel, dim3(1), dim3(kCombineThreads), 0, s, part, n_rows, P,
                     one_wg ? 1 : 0, H, argmax, p1, D, nD, maxD, tau, e_max, flag);
  return hipGetLastError();
}

}  // namespace ec
