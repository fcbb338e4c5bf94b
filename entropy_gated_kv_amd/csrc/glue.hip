// Step glue: embedding gather of the selected rows and RMSNorm.  (The decode
// and decision kernel, which unmasks tokens, appends to the decode history
// and takes the threshold decision, runs with the entropy pass in
// entropy.hip.)
#include <math.h>

#include "ec_device.h"
#include "ec_launch.h"

namespace ec {

namespace {

constexpr int kEmbedWgPerCu = 8;

// 16-byte vectors of a storage type, as floats
template <typename T> struct Vec16;
template <> struct Vec16<float> {
  static constexpr int N = 4;
  __device__ static void unpack(const u32x4& v, float (&f)[4]) {
#pragma unroll
    for (int i = 0; i < 4; ++i) f[i] = __uint_as_float(v[i]);
  }
  __device__ static u32x4 pack(const float (&f)[4]) {
    return u32x4{__float_as_uint(f[0]), __float_as_uint(f[1]), __float_as_uint(f[2]), __float_as_uint(f[3])};
  }
};
template <> struct Vec16<bf16_t> {
  static constexpr int N = 8;
  __device__ static void unpack(const u32x4& v, float (&f)[8]) {
#pragma unroll
    for (int i = 0; i < 4; ++i) { f[2 * i] = bf16_lo(v[i]); f[2 * i + 1] = bf16_hi(v[i]); }
  }
  __device__ static u32x4 pack(const float (&f)[8]) {
    return u32x4{pack_bf16x2(f[0], f[1]), pack_bf16x2(f[2], f[3]), pack_bf16x2(f[4], f[5]), pack_bf16x2(f[6], f[7])};
  }
};

// x[r, :] = tok_emb[tokens[rows[r]], :] + pos_emb[rows[r], :] (fp32 add, one
// rounding): a workgroup per row, 16-byte vectors (d is a multiple of the
// vector width).  The grid is at most kEmbedWgPerCu per CU, so a partial step
// of a long sequence does not dispatch a workgroup per cache row.
template <typename T>
__global__ __launch_bounds__(256) void embed_kernel(const T* __restrict__ tok_emb,
                                                   const T* __restrict__ pos_emb,
                                                   const int32_t* __restrict__ tokens,
                                                   const int32_t* __restrict__ rows,
                                                   const int32_t* __restrict__ n_rows, int d,
                                                   T* __restrict__ x) {
  using V = Vec16<T>;
  const int n = *n_rows;
  for (int r = blockIdx.x; r < n; r += gridDim.x) {     // the grid is capped; rows stride over it
    const int p = rows[r];
    const int t = tokens[p];
    const u32x4* te = reinterpret_cast<const u32x4*>(tok_emb + int64_t(t) * d);
    const u32x4* pe = reinterpret_cast<const u32x4*>(pos_emb + int64_t(p) * d);
    u32x4* xr = reinterpret_cast<u32x4*>(x + int64_t(r) * d);
    for (int v = threadIdx.x; v < d / V::N; v += 256) {
      float a[V::N], b[V::N];
      V::unpack(te[v], a);
      V::unpack(pe[v], b);
#pragma unroll
      for (int i = 0; i < V::N; ++i) a[i] += b[i];
      xr[v] = V::pack(a);
    }
  }
}

// out[r, :] = x[r, :] / sqrt(mean(x[r, :]^2) + eps) * gain   (one workgroup per row)
// The row and the gain are loaded once, as 16-byte vectors, and kept in
// registers across the reduction (rows up to kNormKeep * 256 vectors; wider
// rows re-read the rest).
constexpr int kNormKeep = 4;

template <typename T>
__global__ __launch_bounds__(256) void rmsnorm_kernel(const T* __restrict__ x,
                                                     const int32_t* __restrict__ n_rows, int d,
                                                     const T* __restrict__ gain, float eps,
                                                     T* __restrict__ out) {
  using V = Vec16<T>;
  const int r = blockIdx.x;
  if (r >= *n_rows) return;
  const int nv = d / V::N;
  const u32x4* xr = reinterpret_cast<const u32x4*>(x + int64_t(r) * d);
  const u32x4* gr = reinterpret_cast<const u32x4*>(gain);
  u32x4 xv[kNormKeep], gv[kNormKeep];
#pragma unroll
  for (int i = 0; i < kNormKeep; ++i) {
    const int v = threadIdx.x + i * 256;
    if (v < nv) { xv[i] = xr[v]; gv[i] = gr[v]; }
  }
  float ss = 0.f;
#pragma unroll
  for (int i = 0; i < kNormKeep; ++i) {
    if (threadIdx.x + i * 256 >= nv) break;
    float f[V::N];
    V::unpack(xv[i], f);
#pragma unroll
    for (int e = 0; e < V::N; ++e) ss = fmaf(f[e], f[e], ss);
  }
  for (int v = threadIdx.x + kNormKeep * 256; v < nv; v += 256) {
    float f[V::N];
    V::unpack(xr[v], f);
#pragma unroll
    for (int e = 0; e < V::N; ++e) ss = fmaf(f[e], f[e], ss);
  }
  ss = wave_sum(ss);
  __shared__ float sw[4];
  if ((threadIdx.x & 63) == 0) sw[threadIdx.x >> 6] = ss;
  __syncthreads();
  const float tot = (sw[0] + sw[1]) + (sw[2] + sw[3]);
  const float inv = 1.0f / sqrtf(tot / float(d) + eps);
  u32x4* orow = reinterpret_cast<u32x4*>(out + int64_t(r) * d);
  auto scaled = [&](const u32x4& xw, const u32x4& gw) {
    float a[V::N], g[V::N];
    V::unpack(xw, a);
    V::unpack(gw, g);
#pragma unroll
    for (int e = 0; e < V::N; ++e) a[e] = a[e] * inv * g[e];
    return V::pack(a);
  };
#pragma unroll
  for (int i = 0; i < kNormKeep; ++i) {
    const int v = threadIdx.x + i * 256;
    if (v < nv) orow[v] = scaled(xv[i], gv[i]);
  }
  for (int v = threadIdx.x + kNormKeep * 256; v < nv; v += 256) orow[v] = scaled(xr[v], gr[v]);
}

}  // namespace

hipError_t launch_embed(int dtype, const void* tok_emb, const void* pos_emb, const int32_t* tokens,
                        const int32_t* rows, const int32_t* n_rows, int max_rows, int d, void* x,
                        hipStream_t s) {
  const int cap = kEmbedWgPerCu * device_cu_count();
  max_rows = max_rows < cap ? max_rows : cap;
  if (dtype == 1)
    hipLaunchKernelGGL(embed_kernel<bf16_t>, dim3(max_rows), dim3(256), 0, s,
                       static_cast<const bf16_t*>(tok_emb), static_cast<const bf16_t*>(pos_emb),
                       tokens, rows, n_rows, d, static_cast<bf16_t*>(x));
  else
    hipLaunchKernelGGL(embed_kernel<float>, dim3(max_rows), dim3(256), 0, s,
                       static_cast<const float*>(tok_emb), static_cast<const float*>(pos_emb),
                       tokens, rows, n_rows, d, static_cast<float*>(x));
  return hipGetLastError();
}

hipError_t launch_rmsnorm(int dtype, const void* x, const int32_t* n_rows, int max_rows, int d,
                          const void* gain, float eps, void* out, hipStream_t s) {
  if (dtype == 1)
    hipLaunchKernelGGL(rmsnorm_kernel<bf16_t>, dim3(max_rows), dim3(256), 0, s,
                       static_cast<const bf16_t*>(x), n_rows, d, static_cast<const bf16_t*>(gain),
                       eps, static_cast<bf16_t*>(out));
  else
    hipLaunchKernelGGL(rmsnorm_kernel<float>, dim3(max_rows), dim3(256), 0, s,
                       static_cast<const float*>(x), n_rows, d, static_cast<const float*>(gain), eps,
                       static_cast<float*>(out));
  return hipGetLastError();
}

}  // namespace ec
