// Device-side helpers shared by the gfx950 kernels (wave64, MFMA operand types,
// bfloat16 conversions, wave reductions).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ec {

constexpr int kWave = 64;

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// Storage element types: float, or bfloat16 kept as raw 16-bit patterns.
struct bf16_t { uint16_t bits; };

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }
__device__ __forceinline__ float bf16_to_f32(uint16_t b) { return __uint_as_float(uint32_t(b) << 16); }

// float -> bfloat16, round to nearest even (v_cvt_pk_bf16_f32); NaN stays NaN.
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  return __builtin_bit_cast(uint16_t, static_cast<__bf16>(f));
}
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return uint32_t(f32_to_bf16(lo)) | (uint32_t(f32_to_bf16(hi)) << 16);
}

template <typename T> struct Elem;
template <> struct Elem<float> {
  static constexpr int kPerVec = 4;   // elements per 16-byte vector
  __device__ static float load(const float* p, int64_t i) { return p[i]; }
  __device__ static void store(float* p, int64_t i, float v) { p[i] = v; }
};
template <> struct Elem<bf16_t> {
  static constexpr int kPerVec = 8;
  __device__ static float load(const bf16_t* p, int64_t i) { return bf16_to_f32(p[i].bits); }
  __device__ static void store(bf16_t* p, int64_t i, float v) { p[i].bits = f32_to_bf16(v); }
};

// Unpack one 16-byte vector into floats.
__device__ __forceinline__ void unpack16(const u32x4& v, float (&x)[8]) {
  x[0] = bf16_lo(v.x); x[1] = bf16_hi(v.x); x[2] = bf16_lo(v.y); x[3] = bf16_hi(v.y);
  x[4] = bf16_lo(v.z); x[5] = bf16_hi(v.z); x[6] = bf16_lo(v.w); x[7] = bf16_hi(v.w);
}
__device__ __forceinline__ void unpack16(const f32x4& v, float (&x)[4]) {
  x[0] = v.x; x[1] = v.y; x[2] = v.z; x[3] = v.w;
}

// Wave64 reductions with DPP (no LDS traffic): pairs, quads, half-rows, rows of
// 16, then row_bcast:15 / row_bcast:31 fold rows 0-2 into row 3; the total
// lands in lane 63 and is read back with readlane.  The order is fixed, so
// float sums are deterministic.  Lanes a DPP step does not write keep `old`.
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ int dpp_i(int old, int src) {
  return __builtin_amdgcn_update_dpp(old, src, CTRL, ROW_MASK, 0xf, false);
}
__device__ __forceinline__ float wave_sum_dpp(float v) {
  int x = __float_as_int(v);
  v += __int_as_float(dpp_i<0xB1, 0xf>(0, x)); x = __float_as_int(v);   // quad_perm [1,0,3,2]
  v += __int_as_float(dpp_i<0x4E, 0xf>(0, x)); x = __float_as_int(v);   // quad_perm [2,3,0,1]
  v += __int_as_float(dpp_i<0x141, 0xf>(0, x)); x = __float_as_int(v);  // row_half_mirror
  v += __int_as_float(dpp_i<0x140, 0xf>(0, x)); x = __float_as_int(v);  // row_mirror
  v += __int_as_float(dpp_i<0x142, 0xa>(0, x)); x = __float_as_int(v);  // row_bcast:15
  v += __int_as_float(dpp_i<0x143, 0xc>(0, x)); x = __float_as_int(v);  // row_bcast:31
  return __int_as_float(__builtin_amdgcn_readlane(x, 63));
}
// NaN-propagating maximum (v_maximum_f32: no input canonicalisation).
__device__ __forceinline__ float wave_max_dpp(float v) {
  int x = __float_as_int(v);
  v = __builtin_elementwise_maximum(v, __int_as_float(dpp_i<0xB1, 0xf>(x, x))); x = __float_as_int(v);
  v = __builtin_elementwise_maximum(v, __int_as_float(dpp_i<0x4E, 0xf>(x, x))); x = __float_as_int(v);
  v = __builtin_elementwise_maximum(v, __int_as_float(dpp_i<0x141, 0xf>(x, x))); x = __float_as_int(v);
  v = __builtin_elementwise_maximum(v, __int_as_float(dpp_i<0x140, 0xf>(x, x))); x = __float_as_int(v);
  v = __builtin_elementwise_maximum(v, __int_as_float(dpp_i<0x142, 0xa>(x, x))); x = __float_as_int(v);
  v = __builtin_elementwise_maximum(v, __int_as_float(dpp_i<0x143, 0xc>(x, x))); x = __float_as_int(v);
  return __int_as_float(__builtin_amdgcn_readlane(x, 63));
}
__device__ __forceinline__ int wave_min_i_dpp(int v) {
  v = min(v, dpp_i<0xB1, 0xf>(v, v));
  v = min(v, dpp_i<0x4E, 0xf>(v, v));
  v = min(v, dpp_i<0x141, 0xf>(v, v));
  v = min(v, dpp_i<0x140, 0xf>(v, v));
  v = min(v, dpp_i<0x142, 0xa>(v, v));
  v = min(v, dpp_i<0x143, 0xc>(v, v));
  return __builtin_amdgcn_readlane(v, 63);
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, kWave));
  return v;
}
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, kWave);
  return v;
}
__device__ __forceinline__ int wave_sum_i(int v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, kWave);
  return v;
}

// ---- global -> LDS copies (gfx950 global_load_lds_dwordx4)
// One 1-KiB copy: lane l's 16 bytes at sbase + voff land at LDS byte
// lds + 16 l.  M0 (the LDS base of the copy) is saved and restored.  The
// copies are not visible to the compiler's wait tracking: callers wait with
// wait_copies_and_sync<N>() (or wait_groups_and_sync) before reading what
// they wrote, and must issue no other vector memory operation in between
// whose completion they rely on.
__device__ __forceinline__ void lds_copy16(const void* sbase, uint32_t voff, uint32_t lds) {
  uint32_t save;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %1\n\t"
      "global_load_lds_dwordx4 %2, %3\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(save)
      : "s"(lds), "v"(voff), "s"(sbase)
      : "memory");
}
// Wait until at most N of this wave's copies are in flight, then synchronise
// the workgroup; the empty asm statements keep LDS reads on their side.
template <int N>
__device__ __forceinline__ void wait_copies_and_sync() {
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}
// Copies are issued in groups of PER (one pipeline stage per wave): wait until
// at most `younger` (0..2) groups issued after the one needed are in flight.
template <int PER>
__device__ __forceinline__ void wait_groups_and_sync(int younger) {
  if (younger >= 2) wait_copies_and_sync<2 * PER>();
  else if (younger == 1) wait_copies_and_sync<PER>();
  else wait_copies_and_sync<0>();
}
// LDS byte address of a dynamic LDS block (the copies take it in M0)
__device__ __forceinline__ uint32_t lds_addr(const char* p) {
  return uint32_t(size_t((__attribute__((address_space(3))) const char*)(p)));
}

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

}  // namespace ec
