// Row GEMM with fused epilogues: C[r, n] = sum_k A[row(r), k] * W[n, k] for the
// selected rows r < *n_rows (device count), on MFMA.
//
// This is the projection work of one denoising step: the selective QKV refresh
// with its scatter into the KV cache (EntropyCache, Chinese summary page §2.2:
// only the selected rows are recomputed; the rest of the cache is reused), the
// output projection and FFN with residual adds, and the LM head over the
// block's masked rows.
//
// Two tilings, both launched; each reads the row count from device memory and
// the one that does not apply exits at once, so no row count crosses to the
// host:
//  * skinny (n <= 128, partial steps and the LM head): weights are streamed
//    from HBM exactly once across the grid.  A workgroup owns 128 or 256
//    output columns (32 or 64 per wave) and a K range; the selected rows' A
//    slice is staged in LDS (double-buffered, 64 k per stage) and shared by the
//    four waves; W fragments go global -> registers, one iteration ahead.  When
//    the column tiles alone cannot fill the chip the K range is split over
//    workgroups; the last workgroup of a tile sums the partials in split order
//    (deterministic) and runs the epilogue.
//  * tiled (n > 128, full steps): 128 x 128 output tiles, 64 k per stage,
//    A and W tiles double-buffered in LDS, 2 x 2 waves of 64 x 64.
// MFMA: v_mfma_f32_32x32x16_bf16 (bf16) or v_mfma_f32_32x32x2_f32 (fp32), fp32
// accumulation.  Each lane's 16-byte loads cover consecutive k; the k order
// inside an MFMA is permuted identically for A and W, which leaves the sum
// unchanged.
#include <math.h>

#include "ec_device.h"
#include "ec_launch.h"

namespace ec {

namespace {

constexpr int kThreads = 256;
constexpr int kSkinnyMaxRows = 128;

template <typename T> struct Mma;
template <> struct Mma<bf16_t> {
  typedef bf16x8 Frag;
  __device__ static void run(f32x16& acc, const u32x4& a, const u32x4& b) {
    acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                  __builtin_bit_cast(bf16x8, b), acc, 0, 0, 0);
  }
};
template <> struct Mma<float> {
  __device__ static void run(f32x16& acc, const u32x4& a, const u32x4& b) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
      acc = __builtin_amdgcn_mfma_f32_32x32x2f32(__uint_as_float(a[i]), __uint_as_float(b[i]), acc,
                                                 0, 0, 0);
  }
};

// Per-lane vectors per lane-half per iteration: 4 x 16 B = 64 consecutive bytes of k.
constexpr int kVecs = 4;
template <typename T> constexpr int kit() { return 2 * kVecs * (16 / int(sizeof(T))); }  // k per iteration

struct GP {
  const void* A;
  int64_t lda;
  const int32_t* a_idx;
  const int32_t* n_rows;
  int max_rows;
  const void* W;
  const void* W2;
  int N, K;
  void* C;
  int64_t ldc;
  int epi;
  const int32_t* rows;
  void* q;
  void* kc;
  void* vc;
  int Hq, Hkv, dh, L_cap;
  const float* scale;
  const int32_t* scale_pos;
  float* part;       // split-K partials
  int S;             // K splits (skinny)
  int KS;            // k per split
};

__device__ __forceinline__ float silu(float g) { return g / (1.0f + __expf(-g)); }

template <typename T, int EPI>
__device__ __forceinline__ void epilogue(const GP& p, int r, int n, float v, float v2) {
  T* C = static_cast<T*>(p.C);
  if constexpr (EPI == int(Epi::kStore)) {
    Elem<T>::store(C, int64_t(r) * p.ldc + n, v);
  } else if constexpr (EPI == int(Epi::kResidual)) {
    const int64_t i = int64_t(r) * p.ldc + n;
    Elem<T>::store(C, i, Elem<T>::load(C, i) + v);
  } else if constexpr (EPI == int(Epi::kSwiGLU)) {
    Elem<T>::store(C, int64_t(r) * p.ldc + n, silu(v) * v2);
  } else if constexpr (EPI == int(Epi::kLogits)) {
    const float s = (p.scale != nullptr) ? p.scale[p.scale_pos[r]] : 1.0f;
    Elem<T>::store(C, int64_t(r) * p.ldc + n, v * s);
  } else {  // kQKV: Q compact, K cache row-major, V cache transposed
    const int qc = p.Hq * p.dh, kc = (p.Hq + p.Hkv) * p.dh;
    if (n < qc) {
      Elem<T>::store(static_cast<T*>(p.q), int64_t(r) * qc + n, v);
    } else if (n < kc) {
      const int g = (n - qc) / p.dh, e = (n - qc) - g * p.dh;
      Elem<T>::store(static_cast<T*>(p.kc), (int64_t(g) * p.L_cap + p.rows[r]) * p.dh + e, v);
    } else {
      const int g = (n - kc) / p.dh, e = (n - kc) - g * p.dh;
      Elem<T>::store(static_cast<T*>(p.vc), (int64_t(g) * p.dh + e) * p.L_cap + p.rows[r], v);
    }
  }
}

// 32x32 accumulator element j of lane l: row 8*(j/4) + 4*(l/32) + j%4, column l%32.
__device__ __forceinline__ int acc_row(int j, int lane) { return 8 * (j >> 2) + 4 * (lane >> 5) + (j & 3); }

// ============================================================================ skinny
// Floats of one split's partial tile, laid out [element][thread] and sized for
// four row blocks: element (rb, cb, j) of thread t at ((rb*CB + cb)*16 + j)*256 + t,
// the second accumulator (DUAL) after 4*CB*16 elements.
template <int CB, bool DUAL>
__host__ __device__ constexpr int split_chunk() { return 4 * CB * 16 * (DUAL ? 2 : 1) * kThreads; }

template <typename T, int MB, int CB, bool DUAL, int EPI>
__device__ __forceinline__ void skinny_body(const GP& p, int n_rows, char* smem) {
  constexpr int VPL = 16 / int(sizeof(T));
  constexpr int KIT = kit<T>();
  constexpr int ROWB = KIT * int(sizeof(T)) + 16;           // LDS row pitch (bytes), padded
  constexpr int NT = 4 * CB * 32;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, h = lane >> 5;
  const int b = blockIdx.x;
  const int split = b % p.S, tile = b / p.S;
  const int k0 = split * p.KS;
  const int k1 = min(p.K, k0 + p.KS);
  const int nit = (k1 - k0) / KIT;
  const int col0 = tile * NT + wave * CB * 32;

  const T* A = static_cast<const T*>(p.A);
  const T* W = static_cast<const T*>(p.W);
  const T* W2 = static_cast<const T*>(p.W2);

  // A staging: MB*32 rows x KIT k per stage; 16 B per thread-load.
  constexpr int AV = MB * 32 * (KIT / VPL);                  // 16-B vectors per stage
  constexpr int APT = (AV + kThreads - 1) / kThreads;        // per thread
  u32x4 areg[APT];
  auto a_load = [&](int it) {
#pragma unroll
    for (int i = 0; i < APT; ++i) {
      const int v = tid + i * kThreads;
      const int r = v / (KIT / VPL), c = v % (KIT / VPL);
      u32x4 x = {0u, 0u, 0u, 0u};
      if (v < AV && r < n_rows) {
        const int ar = (p.a_idx != nullptr) ? p.a_idx[r] : r;
        x = *reinterpret_cast<const u32x4*>(A + int64_t(ar) * p.lda + k0 + it * KIT + c * VPL);
      }
      areg[i] = x;
    }
  };
  auto a_store = [&](int buf) {
    char* base = smem + buf * (MB * 32 * ROWB);
#pragma unroll
    for (int i = 0; i < APT; ++i) {
      const int v = tid + i * kThreads;
      if (v < AV) {
        const int r = v / (KIT / VPL), c = v % (KIT / VPL);
        *reinterpret_cast<u32x4*>(base + r * ROWB + c * 16) = areg[i];
      }
    }
  };

  // W fragments: per column block, kVecs consecutive 16-B vectors of row n.
  u32x4 wcur[CB][kVecs], wnext[CB][kVecs];
  u32x4 w2cur[DUAL ? CB : 1][kVecs], w2next[DUAL ? CB : 1][kVecs];
  auto w_load = [&](u32x4 (&dst)[CB][kVecs], const T* Wm, int it) {
#pragma unroll
    for (int cb = 0; cb < CB; ++cb) {
      const int n = col0 + cb * 32 + (lane & 31);
      const T* src = Wm + int64_t(min(n, p.N - 1)) * p.K + k0 + it * KIT + h * kVecs * VPL;
#pragma unroll
      for (int v = 0; v < kVecs; ++v) dst[cb][v] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(src) + v);
    }
  };

  f32x16 acc[MB][CB], acc2[DUAL ? MB : 1][DUAL ? CB : 1];
#pragma unroll
  for (int rb = 0; rb < MB; ++rb)
#pragma unroll
    for (int cb = 0; cb < CB; ++cb) {
      acc[rb][cb] = f32x16{};
      if constexpr (DUAL) acc2[rb][cb] = f32x16{};
    }

  if (nit > 0) {
    a_load(0);
    w_load(wcur, W, 0);
    if constexpr (DUAL) w_load(w2cur, W2, 0);
    a_store(0);
  }
  __syncthreads();
  for (int it = 0; it < nit; ++it) {
    const bool more = (it + 1 < nit);
    if (more) {
      a_load(it + 1);
      w_load(wnext, W, it + 1);
      if constexpr (DUAL) w_load(w2next, W2, it + 1);
    }
    const char* base = smem + (it & 1) * (MB * 32 * ROWB);
#pragma unroll
    for (int v = 0; v < kVecs; ++v) {
#pragma unroll
      for (int rb = 0; rb < MB; ++rb) {
        const u32x4 a = *reinterpret_cast<const u32x4*>(base + (rb * 32 + (lane & 31)) * ROWB +
                                                        (h * kVecs + v) * 16);
#pragma unroll
        for (int cb = 0; cb < CB; ++cb) {
          Mma<T>::run(acc[rb][cb], a, wcur[cb][v]);
          if constexpr (DUAL) Mma<T>::run(acc2[rb][cb], a, w2cur[cb][v]);
        }
      }
    }
    if (more) {
      a_store((it + 1) & 1);
#pragma unroll
      for (int cb = 0; cb < CB; ++cb)
#pragma unroll
        for (int v = 0; v < kVecs; ++v) {
          wcur[cb][v] = wnext[cb][v];
          if constexpr (DUAL) w2cur[cb][v] = w2next[cb][v];
        }
    }
    __syncthreads();
  }

  // ---- split-K: publish this split's partial tile; gemm_splitk_epilogue sums
  // the splits in order and runs the epilogue (no cross-workgroup fence).
  if (p.S > 1) {
    float* mine = p.part + (int64_t(tile) * p.S + split) * split_chunk<CB, DUAL>();
#pragma unroll
    for (int rb = 0; rb < MB; ++rb)
#pragma unroll
      for (int cb = 0; cb < CB; ++cb)
#pragma unroll
        for (int j = 0; j < 16; ++j) {
          mine[((rb * CB + cb) * 16 + j) * kThreads + tid] = acc[rb][cb][j];
          if constexpr (DUAL)
            mine[((4 * CB) * 16 + (rb * CB + cb) * 16 + j) * kThreads + tid] = acc2[rb][cb][j];
        }
    return;
  }

  // ---- epilogue
#pragma unroll
  for (int rb = 0; rb < MB; ++rb)
#pragma unroll
    for (int cb = 0; cb < CB; ++cb) {
      const int n = col0 + cb * 32 + (lane & 31);
      if (n >= p.N) continue;
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        const int r = rb * 32 + acc_row(j, lane);
        if (r < n_rows) epilogue<T, EPI>(p, r, n, acc[rb][cb][j], DUAL ? acc2[DUAL ? rb : 0][DUAL ? cb : 0][j] : 0.f);
      }
    }
}

// MBX: largest row-block count this launch can see (from max_rows on the host);
// the kernel picks the body for the device row count.
template <typename T, int MBX, int CB, bool DUAL, int EPI>
__global__ __launch_bounds__(kThreads) void gemm_skinny_kernel(GP p) {
  extern __shared__ __attribute__((aligned(16))) char smem[];
  const int n_rows = min(*p.n_rows, p.max_rows);
  if (n_rows <= 0 || n_rows > kSkinnyMaxRows) return;
  const int mb = (n_rows + 31) / 32;
  if (mb == 1 || MBX == 1) skinny_body<T, 1, CB, DUAL, EPI>(p, n_rows, smem);
  else if constexpr (MBX >= 2) {
    if (mb == 2 || MBX == 2) skinny_body<T, 2, CB, DUAL, EPI>(p, n_rows, smem);
    else if constexpr (MBX >= 3) {
      if (mb == 3 || MBX == 3) skinny_body<T, 3, CB, DUAL, EPI>(p, n_rows, smem);
      else if constexpr (MBX >= 4) skinny_body<T, 4, CB, DUAL, EPI>(p, n_rows, smem);
    }
  }
}

// Sum the S partial tiles of each column tile in split order, then epilogue.
template <typename T, int CB, bool DUAL, int EPI>
__global__ __launch_bounds__(kThreads) void gemm_splitk_epilogue(GP p) {
  const int n_rows = min(*p.n_rows, p.max_rows);
  if (n_rows <= 0 || n_rows > kSkinnyMaxRows) return;
  const int mb = (n_rows + 31) / 32;
  const int tile = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  constexpr int NT = 4 * CB * 32;
  const float* base = p.part + int64_t(tile) * p.S * split_chunk<CB, DUAL>();
  for (int rb = 0; rb < mb; ++rb)
#pragma unroll
    for (int cb = 0; cb < CB; ++cb) {
      const int n = tile * NT + wave * CB * 32 + cb * 32 + (lane & 31);
#pragma unroll 4
      for (int j = 0; j < 16; ++j) {
        const int r = rb * 32 + acc_row(j, lane);
        const int e = ((rb * CB + cb) * 16 + j) * kThreads + tid;
        float v = 0.f, v2 = 0.f;
        for (int s = 0; s < p.S; ++s) {
          v += base[int64_t(s) * split_chunk<CB, DUAL>() + e];
          if constexpr (DUAL) v2 += base[int64_t(s) * split_chunk<CB, DUAL>() + (4 * CB) * 16 * kThreads + e];
        }
        if (r < n_rows && n < p.N) epilogue<T, EPI>(p, r, n, v, v2);
      }
    }
}

// ============================================================================ tiled
constexpr int kBM = 128, kBN = 128;

template <typename T, bool DUAL, int EPI>
__global__ __launch_bounds__(kThreads) void gemm_tiled_kernel(GP p) {
  constexpr int VPL = 16 / int(sizeof(T));
  constexpr int KIT = kit<T>();
  constexpr int ROWB = KIT * int(sizeof(T)) + 16;
  constexpr int NB = DUAL ? 2 : 1;                       // weight matrices
  extern __shared__ __attribute__((aligned(16))) char smem[];
  const int n_rows = min(*p.n_rows, p.max_rows);
  if (n_rows <= kSkinnyMaxRows) return;                  // the skinny kernel handles it
  const int tiles_m = (p.max_rows + kBM - 1) / kBM;
  const int tiles_n = (p.N + kBN - 1) / kBN;
  // XCD-aware order: consecutive workgroups land on different XCDs; give each
  // XCD a contiguous run of tiles (row tiles fastest) so a weight tile is shared in L2.
  const int total = tiles_m * tiles_n;
  const int b = blockIdx.x;
  const int per_xcd = (total + 7) / 8;
  const int t = (b % 8) * per_xcd + b / 8;
  if (t >= total) return;
  const int tm = t % tiles_m, tn = t / tiles_m;
  const int row0 = tm * kBM, col0 = tn * kBN;
  if (row0 >= n_rows) return;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, h = lane >> 5;
  const int wr = (wave >> 1) * 64, wc = (wave & 1) * 64;
  const T* A = static_cast<const T*>(p.A);
  const T* Wm[2] = {static_cast<const T*>(p.W), static_cast<const T*>(p.W2)};

  constexpr int TILEB = kBM * ROWB;                      // bytes of one 128 x KIT tile
  constexpr int STAGE = TILEB * (1 + NB);
  constexpr int VPT = kBM * (KIT / VPL) / kThreads;      // 16-B vectors per thread per tile (4)
  u32x4 ra[VPT], rw[NB][VPT];
  auto g_load = [&](int it) {
    const int kb = it * KIT;
#pragma unroll
    for (int i = 0; i < VPT; ++i) {
      const int v = tid + i * kThreads;
      const int r = v / (KIT / VPL), c = v % (KIT / VPL);
      const int gr = row0 + r;
      u32x4 x = {0u, 0u, 0u, 0u};
      if (gr < n_rows) {
        const int ar = (p.a_idx != nullptr) ? p.a_idx[gr] : gr;
        x = *reinterpret_cast<const u32x4*>(A + int64_t(ar) * p.lda + kb + c * VPL);
      }
      ra[i] = x;
#pragma unroll
      for (int w = 0; w < NB; ++w) {
        const int gn = min(col0 + r, p.N - 1);
        rw[w][i] = *reinterpret_cast<const u32x4*>(Wm[w] + int64_t(gn) * p.K + kb + c * VPL);
      }
    }
  };
  auto s_store = [&](int buf) {
    char* base = smem + buf * STAGE;
#pragma unroll
    for (int i = 0; i < VPT; ++i) {
      const int v = tid + i * kThreads;
      const int r = v / (KIT / VPL), c = v % (KIT / VPL);
      *reinterpret_cast<u32x4*>(base + r * ROWB + c * 16) = ra[i];
#pragma unroll
      for (int w = 0; w < NB; ++w)
        *reinterpret_cast<u32x4*>(base + (1 + w) * TILEB + r * ROWB + c * 16) = rw[w][i];
    }
  };

  f32x16 acc[NB][2][2];
#pragma unroll
  for (int w = 0; w < NB; ++w)
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j) acc[w][i][j] = f32x16{};

  const int nit = p.K / KIT;
  g_load(0);
  s_store(0);
  __syncthreads();
  for (int it = 0; it < nit; ++it) {
    const bool more = (it + 1 < nit);
    if (more) g_load(it + 1);
    const char* base = smem + (it & 1) * STAGE;
#pragma unroll
    for (int v = 0; v < kVecs; ++v) {
      u32x4 a[2], bw[NB][2];
#pragma unroll
      for (int i = 0; i < 2; ++i)
        a[i] = *reinterpret_cast<const u32x4*>(base + (wr + i * 32 + (lane & 31)) * ROWB + (h * kVecs + v) * 16);
#pragma unroll
      for (int w = 0; w < NB; ++w)
#pragma unroll
        for (int j = 0; j < 2; ++j)
          bw[w][j] = *reinterpret_cast<const u32x4*>(base + (1 + w) * TILEB +
                                                     (wc + j * 32 + (lane & 31)) * ROWB + (h * kVecs + v) * 16);
#pragma unroll
      for (int w = 0; w < NB; ++w)
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
          for (int j = 0; j < 2; ++j) Mma<T>::run(acc[w][i][j], a[i], bw[w][j]);
    }
    if (more) s_store((it + 1) & 1);
    __syncthreads();
  }

#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int n = col0 + wc + j * 32 + (lane & 31);
      if (n >= p.N) continue;
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int r = row0 + wr + i * 32 + acc_row(e, lane);
        if (r < n_rows) epilogue<T, EPI>(p, r, n, acc[0][i][j][e], DUAL ? acc[NB - 1][i][j][e] : 0.f);
      }
    }
}

// ---------------------------------------------------------------------------- planning
int mbx_of(int max_rows) { return max_rows >= kSkinnyMaxRows ? 4 : (max_rows + 31) / 32; }

struct Plan {
  int MBX, CB, S, KS, tiles;
  size_t part_floats;
};

template <typename T>
Plan plan_skinny(const GemmArgs& a) {
  Plan pl;
  const bool dual = (a.epi == Epi::kSwiGLU);
  pl.MBX = mbx_of(a.max_rows);
  pl.CB = (dual || a.N <= 1024 || pl.MBX > 2) ? 1 : 2;
  const int NT = 4 * pl.CB * 32;
  pl.tiles = (a.N + NT - 1) / NT;
  const int KIT = kit<T>();
  const int iters = a.K / KIT;
  int S = 1;
  // split K only when the column tiles alone leave most CUs idle, and never for
  // the QKV scatter called without a workspace
  while (pl.tiles * S < 256 && S * 2 <= 16 && iters % (S * 2) == 0 && iters / (S * 2) >= 2) S *= 2;
  pl.S = S;
  pl.KS = (iters / S) * KIT;
  const int CHUNK = 4 * pl.CB * 16 * (dual ? 2 : 1) * kThreads;
  pl.part_floats = (S > 1) ? size_t(pl.tiles) * S * CHUNK : 0;
  return pl;
}

size_t up256(size_t b) { return (b + 255) & ~size_t(255); }

template <typename T, int MBX, int CB, bool DUAL, int EPI>
void go_skinny(dim3 g, size_t lds, hipStream_t s, const GP& p) {
  hipLaunchKernelGGL((gemm_skinny_kernel<T, MBX, CB, DUAL, EPI>), g, dim3(kThreads), lds, s, p);
}

template <typename T, int EPI>
void skinny_by_shape(const Plan& pl, dim3 g, size_t lds, hipStream_t s, const GP& p) {
  if (pl.CB == 2) {                       // CB = 2 only with MBX <= 2
    if (pl.MBX == 1) go_skinny<T, 1, 2, false, EPI>(g, lds, s, p);
    else go_skinny<T, 2, 2, false, EPI>(g, lds, s, p);
  } else {
    switch (pl.MBX) {
      case 1: go_skinny<T, 1, 1, false, EPI>(g, lds, s, p); break;
      case 2: go_skinny<T, 2, 1, false, EPI>(g, lds, s, p); break;
      case 3: go_skinny<T, 3, 1, false, EPI>(g, lds, s, p); break;
      default: go_skinny<T, 4, 1, false, EPI>(g, lds, s, p); break;
    }
  }
}

template <typename T>
hipError_t dispatch_skinny(Epi epi, const Plan& pl, dim3 g, size_t lds, hipStream_t s, const GP& p) {
  switch (epi) {
    case Epi::kStore: skinny_by_shape<T, 0>(pl, g, lds, s, p); break;
    case Epi::kQKV: skinny_by_shape<T, 1>(pl, g, lds, s, p); break;
    case Epi::kResidual: skinny_by_shape<T, 2>(pl, g, lds, s, p); break;
    case Epi::kLogits: skinny_by_shape<T, 4>(pl, g, lds, s, p); break;
    case Epi::kSwiGLU:
      switch (pl.MBX) {
        case 1: go_skinny<T, 1, 1, true, 3>(g, lds, s, p); break;
        case 2: go_skinny<T, 2, 1, true, 3>(g, lds, s, p); break;
        case 3: go_skinny<T, 3, 1, true, 3>(g, lds, s, p); break;
        default: go_skinny<T, 4, 1, true, 3>(g, lds, s, p); break;
      }
      break;
  }
  return hipGetLastError();
}

template <typename T>
hipError_t dispatch_split_epi(Epi epi, const Plan& pl, dim3 g, hipStream_t s, const GP& p) {
  const bool cb2 = (pl.CB == 2);
  switch (epi) {
    case Epi::kStore:
      if (cb2) hipLaunchKernelGGL((gemm_splitk_epilogue<T, 2, false, 0>), g, dim3(kThreads), 0, s, p);
      else hipLaunchKernelGGL((gemm_splitk_epilogue<T, 1, false, 0>), g, dim3(kThreads), 0, s, p);
      break;
    case Epi::kQKV:
      if (cb2) hipLaunchKernelGGL((gemm_splitk_epilogue<T, 2, false, 1>), g, dim3(kThreads), 0, s, p);
      else hipLaunchKernelGGL((gemm_splitk_epilogue<T, 1, false, 1>), g, dim3(kThreads), 0, s, p);
      break;
    case Epi::kResidual:
      if (cb2) hipLaunchKernelGGL((gemm_splitk_epilogue<T, 2, false, 2>), g, dim3(kThreads), 0, s, p);
      else hipLaunchKernelGGL((gemm_splitk_epilogue<T, 1, false, 2>), g, dim3(kThreads), 0, s, p);
      break;
    case Epi::kSwiGLU:
      hipLaunchKernelGGL((gemm_splitk_epilogue<T, 1, true, 3>), g, dim3(kThreads), 0, s, p);
      break;
    case Epi::kLogits:
      if (cb2) hipLaunchKernelGGL((gemm_splitk_epilogue<T, 2, false, 4>), g, dim3(kThreads), 0, s, p);
      else hipLaunchKernelGGL((gemm_splitk_epilogue<T, 1, false, 4>), g, dim3(kThreads), 0, s, p);
      break;
  }
  return hipGetLastError();
}

template <typename T>
hipError_t launch_typed(const GemmArgs& a, void* ws, hipStream_t s, bool allow_split) {
  GP p;
  p.A = a.A; p.lda = a.lda; p.a_idx = a.a_idx; p.n_rows = a.n_rows_dev; p.max_rows = a.max_rows;
  p.W = a.W; p.W2 = a.W2; p.N = a.N; p.K = a.K; p.C = a.C; p.ldc = a.ldc; p.epi = int(a.epi);
  p.rows = a.rows; p.q = a.q_out; p.kc = a.k_cache; p.vc = a.v_cache; p.Hq = a.Hq; p.Hkv = a.Hkv;
  p.dh = a.dh; p.L_cap = a.L_cap; p.scale = a.scale; p.scale_pos = a.scale_pos;
  const bool dual = (a.epi == Epi::kSwiGLU);
  constexpr int KIT = kit<T>();
  constexpr int ROWB = KIT * int(sizeof(T)) + 16;

  Plan pl = plan_skinny<T>(a);
  if (!allow_split || ws == nullptr) { pl.S = 1; pl.KS = a.K; }
  p.S = pl.S; p.KS = pl.KS;
  p.part = static_cast<float*>(ws);
  const size_t lds_sk = size_t(2) * pl.MBX * 32 * ROWB;
  const dim3 g_sk(unsigned(pl.tiles * pl.S));
  hipError_t e = dispatch_skinny<T>(a.epi, pl, g_sk, lds_sk, s, p);
  if (e != hipSuccess) return e;
  if (pl.S > 1) {
    e = dispatch_split_epi<T>(a.epi, pl, dim3(unsigned(pl.tiles)), s, p);
    if (e != hipSuccess) return e;
  }
  if (a.max_rows <= kSkinnyMaxRows) return hipSuccess;

  const int tiles = ((a.max_rows + kBM - 1) / kBM) * ((a.N + kBN - 1) / kBN);
  const unsigned grid = unsigned((tiles + 7) / 8 * 8);
  const size_t lds_t = size_t(2) * kBM * ROWB * (dual ? 3 : 2);
  switch (a.epi) {
    case Epi::kStore: hipLaunchKernelGGL((gemm_tiled_kernel<T, false, 0>), dim3(grid), dim3(kThreads), lds_t, s, p); break;
    case Epi::kQKV: hipLaunchKernelGGL((gemm_tiled_kernel<T, false, 1>), dim3(grid), dim3(kThreads), lds_t, s, p); break;
    case Epi::kResidual: hipLaunchKernelGGL((gemm_tiled_kernel<T, false, 2>), dim3(grid), dim3(kThreads), lds_t, s, p); break;
    case Epi::kSwiGLU: hipLaunchKernelGGL((gemm_tiled_kernel<T, true, 3>), dim3(grid), dim3(kThreads), lds_t, s, p); break;
    case Epi::kLogits: hipLaunchKernelGGL((gemm_tiled_kernel<T, false, 4>), dim3(grid), dim3(kThreads), lds_t, s, p); break;
  }
  return hipGetLastError();
}

}  // namespace

size_t gemm_ws_bytes(const GemmArgs& a) {
  if (a.epi == Epi::kQKV && a.N == 0) return 0;
  Plan pl = (a.dtype == 1) ? plan_skinny<bf16_t>(a) : plan_skinny<float>(a);
  if (pl.S <= 1) return 0;
  return up256(pl.part_floats * 4);
}

hipError_t launch_gemm_rows(const GemmArgs& a, void* ws, hipStream_t s) {
  if (a.N % 32 != 0 || a.K % kit<float>() != 0 || (a.dtype == 1 && a.K % kit<bf16_t>() != 0))
    return hipErrorNotSupported;
  return (a.dtype == 1) ? launch_typed<bf16_t>(a, ws, s, true) : launch_typed<float>(a, ws, s, true);
}

}  // namespace ec
