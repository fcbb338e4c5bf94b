// Bidirectional attention of the selected rows against the whole KV cache.
//
// EntropyCache, Portuguese summary page §1 and Chinese page §1: diffusion LMs
// attend bidirectionally (no causal mask), so every selected query row attends
// to all L cache rows, fresh or stale.  Splitting the cache into partitions
// that are merged afterwards by a log-sum-exp reduction follows the split-KV
// kernel described on the Prefilling-dLLM page (attention-kernel section).
//
// Layout: Q [rows, Hq, dh]; K cache [Hkv, L_cap, dh]; V cache stored
// transposed, [Hkv, dh, L_cap].  Query heads of one KV head are packed into the
// M dimension (packed row rho = r * G + gi, head g * G + gi, G = Hq / Hkv).
//
// Both kernels compute, per 64-row kv tile,
//   S^T = K Q^T        (rows = kv, columns = packed queries)
// so a lane holds one query column and 32 kv scores of each 32-query block:
// the running max and sum need only in-lane work plus one exchange between
// the two wave halves.  K rows are read in a permuted order (bits 2 and 3 of
// the row index swapped) so that each lane's 16 accumulator values of a 32-row
// block are two runs of 8 consecutive kv; those runs are then directly the
// k-operand of
//   O^T += V^T P^T     (A = V^T tile rows from LDS, B = P^T from registers).
//
// bfloat16 (attn_bf16_kernel): each wave owns QB blocks of 32 packed query
// rows, so every K / V^T fragment read from LDS feeds QB MFMAs.  K and V^T
// tiles go from global memory straight into LDS (global_load_lds_dwordx4, no
// register staging) through a ring of NS stages, NS - 1 tiles ahead of the
// compute; the 16-byte chunks of each LDS row are XOR-swizzled so that the
// fragment reads are free of bank conflicts without padding.  In the
// pipelined schedule a wave issues the QK MFMAs of tile t + 1 before the
// softmax of tile t, so the matrix pipe and the vector ALU overlap within the
// wave as well as across the two waves of each SIMD.  P is rounded to bf16 by
// v_cvt_pk_bf16_f32 and its row sums taken with v_dot2_f32_bf16 from the same
// packed values.  The output is rescaled only when a query's running maximum
// grows by more than 2^8 (log2 domain), so P stays <= 256.
// Partial steps (<= 128 selected rows) split the kv range: one workgroup per
// CU, the split count chosen on the device from the actual row count, then a
// log-sum-exp merge kernel.  Full steps run unsplit, their workgroups ordered
// so that each XCD walks the query tiles of the same KV head together.
//
// float32 (attn_kernel, small workloads only): four waves of 32 packed rows,
// K and V^T staged through registers into a double-buffered padded LDS tile.
#include <math.h>

#include "ec_device.h"
#include "ec_launch.h"

namespace ec {

namespace {

constexpr int kThreads = 256;
constexpr int kKV = 64;              // kv rows per tile
constexpr int kQT = 128;             // packed query rows per workgroup
constexpr int kPartialMaxRows = kSmallMaxRows; // rows handled by the split-KV variant

template <typename T, int DH>
struct Geo {
  static constexpr int ES = int(sizeof(T));
  static constexpr int VPL = 16 / ES;                           // elements per 16-B vector
  static constexpr int ROW_BYTES = DH * ES;                     // one K row
  static constexpr int ITERS = ROW_BYTES > 128 ? ROW_BYTES / 128 : 1;
  static constexpr int VH = ROW_BYTES / (32 * ITERS);           // vectors per lane-half per iter
  static constexpr int KPITCH = ROW_BYTES + 16;                 // LDS pitch of a K row
  static constexpr int VPITCH = kKV * ES + 16;                  // LDS pitch of a V^T row
  static constexpr int KTILE = kKV * KPITCH;
  static constexpr int VTILE = DH * VPITCH;
  static constexpr int STAGE = KTILE + VTILE;
  static constexpr int DB = DH / 32;                            // dh blocks of the output
};

template <typename T> struct AttnMma;
template <> struct AttnMma<bf16_t> {
  __device__ static void qk(f32x16& acc, const u32x4& a, const u32x4& b) {
    acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                  __builtin_bit_cast(bf16x8, b), acc, 0, 0, 0);
  }
  // O^T += V^T[rows, kv 8] * P^T[kv 8, q]; vt: 8 values of V^T, p: 8 fp32 probabilities
  __device__ static void pv(f32x16& acc, const char* vt, const float* p) {
    const u32x4 a = *reinterpret_cast<const u32x4*>(vt);
    u32x4 b;
    b.x = pack_bf16x2(p[0], p[1]); b.y = pack_bf16x2(p[2], p[3]);
    b.z = pack_bf16x2(p[4], p[5]); b.w = pack_bf16x2(p[6], p[7]);
    acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                  __builtin_bit_cast(bf16x8, b), acc, 0, 0, 0);
  }
};
template <> struct AttnMma<float> {
  __device__ static void qk(f32x16& acc, const u32x4& a, const u32x4& b) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
      acc = __builtin_amdgcn_mfma_f32_32x32x2f32(__uint_as_float(a[i]), __uint_as_float(b[i]), acc,
                                                 0, 0, 0);
  }
  __device__ static void pv(f32x16& acc, const char* vt, const float* p) {
    const f32x4 a0 = *reinterpret_cast<const f32x4*>(vt);
    const f32x4 a1 = *reinterpret_cast<const f32x4*>(vt + 16);
#pragma unroll
    for (int t = 0; t < 4; ++t) acc = __builtin_amdgcn_mfma_f32_32x32x2f32(a0[t], p[t], acc, 0, 0, 0);
#pragma unroll
    for (int t = 0; t < 4; ++t) acc = __builtin_amdgcn_mfma_f32_32x32x2f32(a1[t], p[4 + t], acc, 0, 0, 0);
  }
};

struct AP {
  const void* q;
  const int32_t* n_rows;
  int max_rows;
  const void* kc;
  const void* vc;
  int L, L_cap, Hq, Hkv, G;
  float sl2;            // scale * log2(e)
  void* out;
  float* opart;         // split partial O   [S][Hkv][Mcap][DH]
  float* mlpart;        // split (m, l)      [S][Hkv][Mcap][2]
  int S;                // kv splits
  int kv_per_split;     // multiple of kKV
  int mcap;             // packed-row capacity of the workspace (partial variant)
  int partial;          // 1: split-KV variant (n <= 128), 0: unsplit (n > 128)
};

// swap bits 2 and 3 of a row index within a 32-row block
__device__ __forceinline__ int perm_row(int x) { return (x & ~12) | ((x & 4) << 1) | ((x & 8) >> 1); }

template <typename T, int DH>
__global__ __launch_bounds__(kThreads) void attn_kernel(AP p) {
  using Gm = Geo<T, DH>;
  extern __shared__ __attribute__((aligned(16))) char smem[];
  const int n = min(*p.n_rows, p.max_rows);
  if (n <= 0) return;
  if (p.partial ? (n > kPartialMaxRows) : (n <= kPartialMaxRows)) return;
  const int M = n * p.G;                                   // packed query rows
  const int qtiles_cap = p.partial ? (kPartialMaxRows * p.G + kQT - 1) / kQT
                                   : (p.max_rows * p.G + kQT - 1) / kQT;
  int b = blockIdx.x;
  const int split = b % p.S; b /= p.S;
  const int qt = b % qtiles_cap;
  const int g = b / qtiles_cap;
  if (qt * kQT >= M) return;
  const int kv0 = split * p.kv_per_split;
  const int kv1 = min(p.L, kv0 + p.kv_per_split);
  if (kv0 >= kv1) return;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, h = lane >> 5;
  const int rho = qt * kQT + wave * 32 + (lane & 31);      // this lane's packed query row
  const bool rho_ok = rho < M;
  const int r = rho_ok ? rho / p.G : 0;
  const int head = g * p.G + (rho_ok ? rho % p.G : 0);
  const T* Q = static_cast<const T*>(p.q);
  const T* Kc = static_cast<const T*>(p.kc) + int64_t(g) * p.L_cap * DH;
  const T* Vc = static_cast<const T*>(p.vc) + int64_t(g) * DH * p.L_cap;

  // Q^T fragments for the whole head dim: [iter][v] 16-B vectors (k-permuted like K)
  u32x4 qf[Gm::ITERS][Gm::VH];
  {
    const char* qrow = reinterpret_cast<const char*>(Q + (int64_t(r) * p.Hq + head) * DH);
#pragma unroll
    for (int it = 0; it < Gm::ITERS; ++it)
#pragma unroll
      for (int v = 0; v < Gm::VH; ++v)
        qf[it][v] = rho_ok ? *reinterpret_cast<const u32x4*>(qrow + it * 128 + (h * Gm::VH + v) * 16)
                           : u32x4{0u, 0u, 0u, 0u};
  }

  // staging of one kv tile: K rows (clamped below L) and V^T columns (zero past L)
  constexpr int KV_VECS = kKV * Gm::ROW_BYTES / 16;        // 16-B vectors of the K tile
  constexpr int VT_VECS = DH * kKV * Gm::ES / 16;           // ... of the V^T tile
  constexpr int KPT = (KV_VECS + kThreads - 1) / kThreads;
  constexpr int VPT = (VT_VECS + kThreads - 1) / kThreads;
  u32x4 rk[KPT], rv[VPT];
  auto g_load = [&](int t0) {
#pragma unroll
    for (int i = 0; i < KPT; ++i) {
      const int v = tid + i * kThreads;
      if (v < KV_VECS) {
        const int row = v / (Gm::ROW_BYTES / 16), c = v % (Gm::ROW_BYTES / 16);
        const int kv = min(t0 + row, p.L - 1);
        rk[i] = *reinterpret_cast<const u32x4*>(reinterpret_cast<const char*>(Kc + int64_t(kv) * DH) + c * 16);
      }
    }
#pragma unroll
    for (int i = 0; i < VPT; ++i) {
      const int v = tid + i * kThreads;
      if (v < VT_VECS) {
        const int e = v / (kKV * Gm::ES / 16), c = v % (kKV * Gm::ES / 16);
        const int kvs = t0 + c * Gm::VPL;                   // first kv of this vector
        u32x4 x = {0u, 0u, 0u, 0u};
        if (kvs < p.L) {
          x = *reinterpret_cast<const u32x4*>(Vc + int64_t(e) * p.L_cap + kvs);
          if (kvs + Gm::VPL > p.L) {                        // zero the columns at or past L
            const int keep = p.L - kvs;                     // elements to keep, 1 .. VPL-1
#pragma unroll
            for (int w = 0; w < 4; ++w) {
              uint32_t m;
              if constexpr (Gm::ES == 2)
                m = (2 * w < keep ? 0x0000ffffu : 0u) | (2 * w + 1 < keep ? 0xffff0000u : 0u);
              else
                m = (w < keep) ? 0xffffffffu : 0u;
              x[w] &= m;
            }
          }
        }
        rv[i] = x;
      }
    }
  };
  auto s_store = [&](int buf) {
    char* base = smem + buf * Gm::STAGE;
#pragma unroll
    for (int i = 0; i < KPT; ++i) {
      const int v = tid + i * kThreads;
      if (v < KV_VECS) {
        const int row = v / (Gm::ROW_BYTES / 16), c = v % (Gm::ROW_BYTES / 16);
        *reinterpret_cast<u32x4*>(base + row * Gm::KPITCH + c * 16) = rk[i];
      }
    }
#pragma unroll
    for (int i = 0; i < VPT; ++i) {
      const int v = tid + i * kThreads;
      if (v < VT_VECS) {
        const int e = v / (kKV * Gm::ES / 16), c = v % (kKV * Gm::ES / 16);
        *reinterpret_cast<u32x4*>(base + Gm::KTILE + e * Gm::VPITCH + c * 16) = rv[i];
      }
    }
  };

  f32x16 o[Gm::DB];
#pragma unroll
  for (int d = 0; d < Gm::DB; ++d) o[d] = f32x16{};
  float m_run = -INFINITY, l_run = 0.f;

  const int ntiles = (kv1 - kv0 + kKV - 1) / kKV;
  g_load(kv0);
  s_store(0);
  __syncthreads();
  for (int t = 0; t < ntiles; ++t) {
    const int t0 = kv0 + t * kKV;
    const bool more = (t + 1 < ntiles);
    if (more) g_load(t0 + kKV);
    const char* base = smem + (t & 1) * Gm::STAGE;

    // ---- S^T = K Q^T for two 32-row kv blocks
    f32x16 s[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      s[kb] = f32x16{};
      const char* krow = base + (kb * 32 + perm_row(lane & 31)) * Gm::KPITCH;
#pragma unroll
      for (int it = 0; it < Gm::ITERS; ++it)
#pragma unroll
        for (int v = 0; v < Gm::VH; ++v) {
          const u32x4 a = *reinterpret_cast<const u32x4*>(krow + it * 128 + (h * Gm::VH + v) * 16);
          AttnMma<T>::qk(s[kb], a, qf[it][v]);
        }
    }
    // ---- online softmax (log2 domain); element i of block kb is kv kb*32 + 16*(i/8) + 8h + i%8
    float tmax = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int kv = t0 + kb * 32 + 16 * (i >> 3) + 8 * h + (i & 7);
        const float v = (kv < kv1) ? s[kb][i] * p.sl2 : -INFINITY;
        s[kb][i] = v;
        tmax = fmaxf(tmax, v);
      }
    tmax = fmaxf(tmax, __shfl_xor(tmax, 32, kWave));
    const float m_new = fmaxf(m_run, tmax);
    const float alpha = (m_new == -INFINITY) ? 1.f : fast_exp2(m_run - m_new);
    const float msub = (m_new == -INFINITY) ? 0.f : m_new;
    float lsum = 0.f;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const float e = fast_exp2(s[kb][i] - msub);
        s[kb][i] = e;
        lsum += e;
      }
    l_run = l_run * alpha + lsum;
    m_run = m_new;
#pragma unroll
    for (int d = 0; d < Gm::DB; ++d)
#pragma unroll
      for (int i = 0; i < 16; ++i) o[d][i] *= alpha;
    // ---- O^T += V^T P^T
#pragma unroll
    for (int d = 0; d < Gm::DB; ++d) {
      const char* vrow = base + Gm::KTILE + (d * 32 + (lane & 31)) * Gm::VPITCH;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          float pv[8];
#pragma unroll
          for (int k = 0; k < 8; ++k) pv[k] = s[kb][8 * j + k];
          AttnMma<T>::pv(o[d], vrow + (kb * 32 + 16 * j + 8 * h) * Gm::ES, pv);
        }
    }
    if (more) s_store((t + 1) & 1);
    __syncthreads();
  }

  const float l_tot = l_run + __shfl_xor(l_run, 32, kWave);
  if (!rho_ok) return;
  // O^T element i of block d: dh row d*32 + 8*(i/4) + 4h + i%4, query column = this lane
  if (!p.partial || p.S == 1) {
    T* O = static_cast<T*>(p.out) + (int64_t(r) * p.Hq + head) * DH;
    const float inv = 1.f / l_tot;
#pragma unroll
    for (int d = 0; d < Gm::DB; ++d)
#pragma unroll
      for (int i = 0; i < 16; ++i) Elem<T>::store(O, d * 32 + 8 * (i >> 2) + 4 * h + (i & 3), o[d][i] * inv);
  } else {
    const int64_t prow = (int64_t(split) * p.Hkv + g) * p.mcap + rho;
    float* op = p.opart + prow * DH;
#pragma unroll
    for (int d = 0; d < Gm::DB; ++d)
#pragma unroll
      for (int i = 0; i < 16; ++i) op[d * 32 + 8 * (i >> 2) + 4 * h + (i & 3)] = o[d][i];
    if (h == 0) { p.mlpart[prow * 2] = m_run; p.mlpart[prow * 2 + 1] = l_tot; }
  }
}

// log-sum-exp merge of the kv splits (split-KV variant only)
template <typename T, int DH>
__global__ __launch_bounds__(256) void attn_merge_kernel(AP p) {
  const int n = min(*p.n_rows, p.max_rows);
  if (n <= 0 || n > kPartialMaxRows) return;
  const int M = n * p.G;
  const int idx = blockIdx.x * 256 + threadIdx.x;          // (g, rho, e)
  const int e = idx % DH;
  const int rho = (idx / DH) % p.mcap;
  const int g = idx / (DH * p.mcap);
  if (g >= p.Hkv || rho >= M) return;
  float mx = -INFINITY;
  for (int s = 0; s < p.S; ++s) {
    const int64_t prow = (int64_t(s) * p.Hkv + g) * p.mcap + rho;
    mx = fmaxf(mx, p.mlpart[prow * 2]);
  }
  float num = 0.f, den = 0.f;
  for (int s = 0; s < p.S; ++s) {
    const int64_t prow = (int64_t(s) * p.Hkv + g) * p.mcap + rho;
    const float ms = p.mlpart[prow * 2];
    if (ms == -INFINITY) continue;                        // empty split
    const float w = fast_exp2(ms - mx);
    num += w * p.opart[prow * DH + e];
    den += w * p.mlpart[prow * 2 + 1];
  }
  const int r = rho / p.G, head = g * p.G + rho % p.G;
  Elem<T>::store(static_cast<T*>(p.out), (int64_t(r) * p.Hq + head) * DH + e, num / den);
}

struct SplitPlan { int S, kvps, mcap; };

SplitPlan plan_split(int L, int Hkv, int G) {
  SplitPlan sp;
  sp.mcap = kPartialMaxRows * G;
  const int qtiles = (sp.mcap + kQT - 1) / kQT;
  const int tiles = (L + kKV - 1) / kKV;
  // enough splits to give the chip two workgroups per CU, but at least 4 kv
  // tiles (256 rows) per split so the partial outputs stay small
  int S = (2 * device_cu_count() + Hkv * qtiles - 1) / (Hkv * qtiles);
  S = max(1, min(S, (tiles + 3) / 4));
  const int per = (tiles + S - 1) / S;                    // kv tiles per split
  sp.kvps = per * kKV;
  sp.S = (tiles + per - 1) / per;
  return sp;
}

template <typename T, int DH>
hipError_t launch_typed(const AttnArgs& a, void* ws, hipStream_t s) {
  using Gm = Geo<T, DH>;
  AP p;
  p.q = a.q; p.n_rows = a.n_rows_dev; p.max_rows = a.max_rows; p.kc = a.k_cache; p.vc = a.v_cache;
  p.L = a.L; p.L_cap = a.L_cap; p.Hq = a.Hq; p.Hkv = a.Hkv; p.G = a.Hq / a.Hkv;
  p.sl2 = a.scale * kLog2e; p.out = a.out;
  const size_t lds = size_t(2) * Gm::STAGE;
  // split-KV variant (n <= 128)
  const SplitPlan sp = plan_split(a.L, a.Hkv, p.G);
  p.S = sp.S; p.kv_per_split = sp.kvps; p.mcap = sp.mcap; p.partial = 1;
  p.opart = static_cast<float*>(ws);
  p.mlpart = p.opart + size_t(sp.S) * a.Hkv * sp.mcap * DH;
  if (sp.S > 1 && ws == nullptr) return hipErrorInvalidValue;
  if (a.paths & kPathSmall) {
    const int qtiles = (kPartialMaxRows * p.G + kQT - 1) / kQT;
    hipLaunchKernelGGL((attn_kernel<T, DH>), dim3(unsigned(a.Hkv * qtiles * sp.S)), dim3(kThreads),
                       lds, s, p);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    if (sp.S > 1) {
      const int64_t total = int64_t(a.Hkv) * sp.mcap * DH;
      hipLaunchKernelGGL((attn_merge_kernel<T, DH>), dim3(unsigned((total + 255) / 256)), dim3(256),
                         0, s, p);
      e = hipGetLastError();
      if (e != hipSuccess) return e;
    }
  }
  if (a.max_rows <= kPartialMaxRows || !(a.paths & kPathLarge)) return hipSuccess;
  // unsplit variant (n > 128)
  p.S = 1; p.kv_per_split = (a.L + kKV - 1) / kKV * kKV; p.partial = 0;
  const int qtiles = (a.max_rows * p.G + kQT - 1) / kQT;
  hipLaunchKernelGGL((attn_kernel<T, DH>), dim3(unsigned(a.Hkv * qtiles)), dim3(kThreads), lds, s, p);
  return hipGetLastError();
}

// ===================================================================== bfloat16

template <int DH, int NW>
struct BG {
  static constexpr int RB = DH * 2;                 // bytes of one K row
  static constexpr int CR = RB / 16;                // 16-byte chunks per K row
  static constexpr int RPW = 256 / RB;              // K rows per 256-byte bank window
  static constexpr int KT = kKV * RB;               // K tile bytes
  static constexpr int VT = DH * kKV * 2;           // V^T tile bytes (DH rows of 128 B)
  static constexpr int STAGE = KT + VT;
  static constexpr int KIW = KT / 1024 / NW;        // 1-KiB copies per wave per K tile
  static constexpr int VIW = VT / 1024 / NW;        // ... per V^T tile
  static constexpr int LOADS = KIW + VIW;           // per wave per tile
  static constexpr int ITERS = RB > 128 ? RB / 128 : 1;
  static constexpr int VH = RB / (32 * ITERS);      // 16-byte vectors per lane half per iteration
  static constexpr int NK = ITERS * VH;             // MFMAs per 32-row kv block (k = DH)
  static constexpr int DB = DH / 32;
  static_assert(KIW >= 1 && VIW >= 1 && KIW * NW * 1024 == KT && VIW * NW * 1024 == VT,
                "the K and V^T tiles split evenly over the waves");
};

// XOR swizzle of the 16-byte chunks of an LDS row: K rows (RB bytes), V^T rows
// (128 bytes).  Consecutive rows of a 32-row fragment read then hit distinct
// 16-byte bank groups.
template <int DH>
__device__ __forceinline__ int swk(int r) { return (r / (256 / (DH * 2))) % (DH / 8); }
__device__ __forceinline__ int swv(int e) { return (e >> 1) & 7; }

// This wave's share of one tile's copies: per-lane source offsets relative to
// the tile start and the kv row / column each lane reads.
template <int DH, int NW>
struct CopyPlan {
  uint32_t koff[BG<DH, NW>::KIW];   // K:   r * RB + chunk * 16
  int kr[BG<DH, NW>::KIW];          //      kv row within the tile
  uint32_t voff[BG<DH, NW>::VIW];   // V^T: (e * L_cap) * 2 + chunk * 16
  int vc[BG<DH, NW>::VIW];          //      first kv of the chunk within the tile
};

template <int DH, int NW>
__device__ __forceinline__ CopyPlan<DH, NW> copy_plan(int L_cap, int wave, int lane) {
  using B = BG<DH, NW>;
  CopyPlan<DH, NW> cp;
#pragma unroll
  for (int i = 0; i < B::KIW; ++i) {
    const int ii = wave * B::KIW + i;
    const int r = ii * (1024 / B::RB) + lane / B::CR;
    const int c = (lane % B::CR) ^ swk<DH>(r);
    cp.kr[i] = r;
    cp.koff[i] = uint32_t(r) * B::RB + uint32_t(c) * 16;
  }
#pragma unroll
  for (int i = 0; i < B::VIW; ++i) {
    const int ii = wave * B::VIW + i;
    const int e = ii * 8 + lane / 8;
    const int c = (lane % 8) ^ swv(e);
    cp.vc[i] = c * 8;
    cp.voff[i] = uint32_t(e) * uint32_t(L_cap) * 2u + uint32_t(c) * 16;
  }
  return cp;
}

// Copy kv tile [t0, t0 + 64) into a stage.  CLAMP (a tile reaching past L):
// K rows clamp to L - 1 and V^T chunks at or past L read chunk 0 of their row
// (finite data, multiplied by P = 0).
template <int DH, int NW, bool CLAMP>
__device__ __forceinline__ void load_tile(const char* kbase, const char* vbase, int L,
                                          const CopyPlan<DH, NW>& cp, int t0, uint32_t stage,
                                          int wave) {
  using B = BG<DH, NW>;
#pragma unroll
  for (int i = 0; i < B::KIW; ++i) {
    uint32_t off = cp.koff[i] + uint32_t(t0) * B::RB;
    if (CLAMP && t0 + cp.kr[i] > L - 1) off -= uint32_t(t0 + cp.kr[i] - (L - 1)) * B::RB;
    lds_copy16(kbase, off, stage + (wave * B::KIW + i) * 1024);
  }
#pragma unroll
  for (int i = 0; i < B::VIW; ++i) {
    uint32_t off = cp.voff[i] + uint32_t(t0) * 2u;
    if (CLAMP && t0 + cp.vc[i] >= L) off -= uint32_t(t0 + cp.vc[i]) * 2u;
    lds_copy16(vbase, off, stage + B::KT + (wave * B::VIW + i) * 1024);
  }
}

// Zero the V^T entries at kv >= L of the stage holding the last tile (the
// cache past L may hold anything, and 0 * NaN would poison the output).
template <int DH, int NW>
__device__ __forceinline__ void zero_vt_tail(char* stage, int t0, int L, int tid) {
  const int x0 = L - t0, cols = kKV - x0;
  for (int q = tid; q < DH * cols; q += NW * kWave) {
    const int e = q / cols, x = x0 + q % cols;
    *reinterpret_cast<uint16_t*>(stage + BG<DH, NW>::KT + e * 128 + (((x >> 3) ^ swv(e)) << 4) +
                                 (x & 7) * 2) = 0;
  }
}

__device__ __forceinline__ f32x16 mfma_bf16(const u32x4& a, const u32x4& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
// two floats -> packed bf16 (v_cvt_pk_bf16_f32: round to nearest even)
__device__ __forceinline__ uint32_t cvt_bf16x2(float lo, float hi) {
  const f32x2 v = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
}
// acc + lo + hi of a packed bf16 pair (v_dot2_f32_bf16 against (1, 1))
__device__ __forceinline__ float add_bf16x2(uint32_t w, float acc) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, w),
                                         __builtin_bit_cast(bf16x2, 0x3f803f80u), acc, false);
}
// lane l's value combined with lane l ^ 32's (v_permlane32_swap returns the
// lower-half value first, the upper-half value second, in every lane)
__device__ __forceinline__ float halves_max(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float halves_sum(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

struct BP {
  const bf16_t* q;
  const int32_t* n_rows;
  int max_rows;
  const bf16_t* kc;
  const bf16_t* vc;
  int L, L_cap, Hq, Hkv, G;
  float sl2;            // scale * log2(e)
  bf16_t* out;
  uint16_t* opart;      // split partial O  [smax][Hkv][mcap][DH], bf16 (unnormalised)
  float* mlpart;        // split (m, l)     [smax][Hkv][mcap][2]
  int mcap;             // packed-row capacity of the split workspace
  int smax;             // split capacity of the split workspace
  int partial;          // 1: split-KV variant (n <= 128), 0: unsplit, 2: the
                        // launch takes either role, by the device row count
  // split-KV variant: the plan, made on the host for a bound nb on the row
  // count (min(max_rows, 128)): qa query tiles, S splits of `per` kv tiles,
  // over the packed rows of nb rows (mb = nb * G)
  int qa, S, per, mb;
  // 1: the split variant is the only one launched (the row count is known to
  // be <= 128), so it starts its loads before the count arrives; 0: it is
  // the gated sibling of the unsplit variant and reads the count first, so
  // that on a full step it exits without loading anything
  int spec;
};

// Split plan of the partial variant for a bound n on the row count: qa query
// tiles, S splits of `per` kv tiles, for `grid` groups.  Made on the host, so
// the kernels can start their loads before the device row count arrives.
struct DPlan { int qa, S, per; };
inline DPlan split_plan(int n, int G, int QT, int Hkv, int tiles, int grid, int smax) {
  DPlan d;
  d.qa = (n * G + QT - 1) / QT;
  int S = grid / (Hkv * d.qa);
  S = max(1, min(S, min(smax, (tiles + 1) / 2)));          // at least two kv tiles per split
  d.per = (tiles + S - 1) / S;
  d.S = (tiles + d.per - 1) / d.per;
  return d;
}

// Work index of a workgroup: the groups one XCD runs (blockIdx = x mod 8) take
// consecutive indices, so they share KV tiles through that XCD's L2.  The
// grid is a multiple of 8, which makes the map a bijection.
__device__ __forceinline__ int xcd_work_index(int b, int grid) { return (b & 7) * (grid >> 3) + (b >> 3); }

// The three phases of one 64-row kv tile for one wave.
//
// S^T = K Q^T: two 32-row kv blocks, each K fragment used QB times.
template <int DH, int QB, int NW>
__device__ __forceinline__ void qk_block(const char* stage, int lane,
                                         const u32x4 (&qf)[QB][BG<DH, NW>::NK], f32x16 (&sc)[QB][2]) {
  using B = BG<DH, NW>;
  const int h = lane >> 5;
#pragma unroll
  for (int kb = 0; kb < 2; ++kb) {
    const int r = kb * 32 + perm_row(lane & 31);
    const char* krow = stage + r * B::RB;
    const int sw = swk<DH>(r);
    u32x4 kf[B::NK];
#pragma unroll
    for (int it = 0; it < B::ITERS; ++it)
#pragma unroll
      for (int v = 0; v < B::VH; ++v)
        kf[it * B::VH + v] =
            *reinterpret_cast<const u32x4*>(krow + (((it * 8 + h * B::VH + v) ^ sw) << 4));
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      f32x16 acc = f32x16{};
#pragma unroll
      for (int k = 0; k < B::NK; ++k) acc = mfma_bf16(kf[k], qf[qb][k], acc);
      sc[qb][kb] = acc;
    }
  }
}

// Online softmax in the log2 domain, branch-free: element i of block kb is kv
// kb*32 + 16*(i/8) + 8h + i%8.  A query's reference maximum m_run moves only
// when the tile's maximum exceeds it by more than 8 (so P <= 2^8); alpha is
// then the factor the output must be scaled by before this tile's P V is
// added (1 otherwise), and the return value says whether any lane needs it.
// TAIL: kv at or past kv1 are masked.
template <int QB, bool TAIL>
__device__ __forceinline__ bool softmax_block(f32x16 (&sc)[QB][2], int t0, int kv1, float sl2, int lane,
                                              float (&m_run)[QB], float (&l_run)[QB], float (&alpha)[QB],
                                              u32x4 (&pf)[QB][2][2]) {
  const int h = lane >> 5;
  bool any = false;
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    if (TAIL) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int i = 0; i < 16; ++i)
          if (t0 + kb * 32 + 16 * (i >> 3) + 8 * h + (i & 7) >= kv1) sc[qb][kb][i] = -INFINITY;
    }
    float mx = sc[qb][0][0];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int i = 0; i < 16; ++i) mx = fmaxf(mx, sc[qb][kb][i]);
    const float mt = halves_max(mx) * sl2;
    const bool need = mt > m_run[qb] + 8.f;                 // false for -inf and NaN
    const float m_new = need ? mt : m_run[qb];
    alpha[qb] = need ? fast_exp2(m_run[qb] - m_new) : 1.f;
    m_run[qb] = m_new;
    any = any || need;
    const float msub = (m_new == -INFINITY) ? 0.f : m_new;
    float ls = l_run[qb] * alpha[qb];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int jj = 0; jj < 2; ++jj) {
        uint32_t w[4];
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          const int i = 8 * jj + 2 * k;
          w[k] = cvt_bf16x2(fast_exp2(fmaf(sc[qb][kb][i], sl2, -msub)),
                            fast_exp2(fmaf(sc[qb][kb][i + 1], sl2, -msub)));
          ls = add_bf16x2(w[k], ls);       // the sum of exactly what the MFMA multiplies
        }
        pf[qb][kb][jj] = u32x4{w[0], w[1], w[2], w[3]};
      }
    l_run[qb] = ls;
  }
  return __ballot(any) != 0;
}

template <int DH, int QB, int NW>
__device__ __forceinline__ void scale_output(const float (&alpha)[QB], f32x16 (&o)[QB][BG<DH, NW>::DB]) {
#pragma unroll
  for (int qb = 0; qb < QB; ++qb)
#pragma unroll
    for (int d = 0; d < BG<DH, NW>::DB; ++d)
#pragma unroll
      for (int i = 0; i < 16; ++i) o[qb][d][i] *= alpha[qb];
}

// O^T += V^T P^T: each V^T fragment used QB times.
template <int DH, int QB, int NW>
__device__ __forceinline__ void pv_block(const char* stage, int lane, const u32x4 (&pf)[QB][2][2],
                                         f32x16 (&o)[QB][BG<DH, NW>::DB]) {
  using B = BG<DH, NW>;
  const int h = lane >> 5;
#pragma unroll
  for (int d = 0; d < B::DB; ++d) {
    const int e = d * 32 + (lane & 31);
    const char* vrow = stage + B::KT + e * 128;
    const int sw = swv(e);
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int jj = 0; jj < 2; ++jj) {
        const u32x4 vf = *reinterpret_cast<const u32x4*>(vrow + (((kb * 4 + jj * 2 + h) ^ sw) << 4));
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) o[qb][d] = mfma_bf16(vf, pf[qb][kb][jj], o[qb][d]);
      }
  }
}

// One whole tile in sequence (the unpipelined schedule).
template <int DH, int QB, int NW, bool TAIL>
__device__ __forceinline__ void attn_tile(const char* stage, int t0, int kv1, float sl2, int lane,
                                          const u32x4 (&qf)[QB][BG<DH, NW>::NK],
                                          f32x16 (&o)[QB][BG<DH, NW>::DB], float (&m_run)[QB],
                                          float (&l_run)[QB]) {
  f32x16 sc[QB][2];
  qk_block<DH, QB, NW>(stage, lane, qf, sc);
  float alpha[QB];
  u32x4 pf[QB][2][2];
  if (softmax_block<QB, TAIL>(sc, t0, kv1, sl2, lane, m_run, l_run, alpha, pf))
    scale_output<DH, QB, NW>(alpha, o);
  pv_block<DH, QB, NW>(stage, lane, pf, o);
}

// PIPE: software-pipelined schedule.  Each step issues the QK MFMAs of tile
// t + 1 before the softmax of tile t, so the matrix pipe works on the next
// tile while the vector ALU exponentiates the current one; the output is then
// rescaled if needed and P V of tile t accumulated.
template <int DH, int QB, int NW, int NS, bool PIPE>
__global__ __launch_bounds__(NW * 64) void attn_bf16_kernel(BP p) {
  static_assert(NS >= 2 && NS <= 4, "two to four LDS stages");
  static_assert(!PIPE || NS >= 3, "the pipelined schedule reads two stages per step");
  using B = BG<DH, NW>;
  constexpr int QT = NW * 32 * QB;                         // packed query rows per workgroup
  extern __shared__ __attribute__((aligned(16))) char smem[];
  // The split variant's work comes from the host plan.  When it is the only
  // variant launched (p.spec), its tile copies and Q loads go out before the
  // row count arrives (one memory latency less) and the count then decides
  // whether the workgroup's rows exist; otherwise, and in the unsplit
  // variant, the count is read first and a workgroup with nothing to do
  // exits before loading anything.
  const int n_dev = *p.n_rows;
  const int j = xcd_work_index(blockIdx.x, gridDim.x);
  const bool part = p.partial == 2 ? min(n_dev, p.max_rows) <= kPartialMaxRows : p.partial != 0;
  int n, M, g, qt, kv0, kv1, split = 0;
  if (part) {
    if (j >= p.Hkv * p.S * p.qa) return;
    qt = j % p.qa;
    split = (j / p.qa) % p.S;
    g = j / (p.qa * p.S);
    kv0 = split * p.per * kKV;
    kv1 = min(p.L, kv0 + p.per * kKV);
    if (kv0 >= kv1) return;
    if (p.spec) {
      M = p.mb;                                             // rows of the plan's bound, for now
      n = 0;
    } else {
      n = min(n_dev, p.max_rows);
      M = n * p.G;
      if (n <= 0 || n > kPartialMaxRows || qt * QT >= M) return;
    }
  } else {
    n = min(n_dev, p.max_rows);
    if (n <= kPartialMaxRows) return;
    M = n * p.G;
    const int qtn = (M + QT - 1) / QT;
    if (j >= p.Hkv * qtn) return;
    qt = j % qtn;
    g = j / qtn;
    kv0 = 0;
    kv1 = p.L;
  }

  const int tid = threadIdx.x, lane = tid & 63, h = lane >> 5;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const char* kbase = reinterpret_cast<const char*>(p.kc + int64_t(g) * p.L_cap * DH);
  const char* vbase = reinterpret_cast<const char*>(p.vc + int64_t(g) * DH * p.L_cap);
  const uint32_t lds0 = lds_addr(smem);
  const int ntiles = (kv1 - kv0 + kKV - 1) / kKV;
  const bool last_partial = kv0 + ntiles * kKV > kv1;      // the last tile reaches past kv1
  const CopyPlan<DH, NW> cp = copy_plan<DH, NW>(p.L_cap, wave, lane);
  auto issue = [&](int t) {                                 // copies of tile t into stage t % NS
    const uint32_t st = lds0 + (t % NS) * B::STAGE;
    if (last_partial && t == ntiles - 1)
      load_tile<DH, NW, true>(kbase, vbase, p.L, cp, kv0 + t * kKV, st, wave);
    else
      load_tile<DH, NW, false>(kbase, vbase, p.L, cp, kv0 + t * kKV, st, wave);
  };

  // the first NS - 1 tiles go out before anything else
#pragma unroll
  for (int t = 0; t < NS - 1; ++t)
    if (t < ntiles) issue(t);

  // Q^T fragments (k-permuted like K): [qb][it * VH + v]
  const int rho0 = qt * QT + wave * 32 * QB;               // first packed row of this wave
  u32x4 qf[QB][B::NK];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const int rho = rho0 + qb * 32 + (lane & 31);
    const bool ok = rho < M;
    const int r = ok ? rho / p.G : 0, head = g * p.G + (ok ? rho % p.G : 0);
    const char* qrow = reinterpret_cast<const char*>(p.q + (int64_t(r) * p.Hq + head) * DH);
#pragma unroll
    for (int it = 0; it < B::ITERS; ++it)
#pragma unroll
      for (int v = 0; v < B::VH; ++v)
        qf[qb][it * B::VH + v] = ok ? *reinterpret_cast<const u32x4*>(qrow + it * 128 + (h * B::VH + v) * 16)
                                    : u32x4{0u, 0u, 0u, 0u};
  }
  if (part && p.spec) {
    // the device row count: a query tile past the rows (or a count outside
    // this variant's range) ends the workgroup once its copies have landed
    n = min(n_dev, p.max_rows);
    M = n * p.G;
    if (n <= 0 || n > kPartialMaxRows || qt * QT >= M) {
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      return;
    }
#pragma unroll
    for (int qb = 0; qb < QB; ++qb)
      if (rho0 + qb * 32 + (lane & 31) >= M)
#pragma unroll
        for (int k = 0; k < B::NK; ++k) qf[qb][k] = u32x4{0u, 0u, 0u, 0u};
  }

  f32x16 o[QB][B::DB];
  float m_run[QB], l_run[QB];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
#pragma unroll
    for (int d = 0; d < B::DB; ++d) o[qb][d] = f32x16{};
    m_run[qb] = -INFINITY;
    l_run[qb] = 0.f;
  }

  if constexpr (PIPE) {
    const bool zero_last = (kv0 + (ntiles - 1) * kKV) + kKV > p.L;   // V^T columns past L in the last tile
    auto stage = [&](int t) { return smem + (t % NS) * B::STAGE; };
    f32x16 scA[QB][2], scB[QB][2];
    // prologue: tile 0 landed, its scores
    wait_groups_and_sync<B::LOADS>(min(NS - 1, ntiles) - 1);
    if (zero_last && ntiles == 1) {
      zero_vt_tail<DH, NW>(stage(0), kv0, p.L, tid);
      __syncthreads();
    }
    qk_block<DH, QB, NW>(stage(0), lane, qf, scA);
    // step t < ntiles - 1: scores of tile t in cur, of tile t + 1 into nxt
    auto step = [&](int t, f32x16 (&cur)[QB][2], f32x16 (&nxt)[QB][2]) {
      wait_groups_and_sync<B::LOADS>(min(NS - 3, ntiles - t - 2));   // tile t + 1 landed
      // stage (t + NS - 1) % NS was last read in step t - 1, which every wave has left
      if (t + NS - 1 < ntiles) issue(t + NS - 1);
      if (zero_last && t + 1 == ntiles - 1) {
        zero_vt_tail<DH, NW>(stage(t + 1), kv0 + (t + 1) * kKV, p.L, tid);
        __syncthreads();
      }
      qk_block<DH, QB, NW>(stage(t + 1), lane, qf, nxt);
      float alpha[QB];
      u32x4 pf[QB][2][2];
      if (softmax_block<QB, false>(cur, kv0 + t * kKV, kv1, p.sl2, lane, m_run, l_run, alpha, pf))
        scale_output<DH, QB, NW>(alpha, o);
      pv_block<DH, QB, NW>(stage(t), lane, pf, o);
    };
    auto finish = [&](f32x16 (&cur)[QB][2]) {               // the last tile
      const int t = ntiles - 1;
      float alpha[QB];
      u32x4 pf[QB][2][2];
      const bool any = last_partial
          ? softmax_block<QB, true>(cur, kv0 + t * kKV, kv1, p.sl2, lane, m_run, l_run, alpha, pf)
          : softmax_block<QB, false>(cur, kv0 + t * kKV, kv1, p.sl2, lane, m_run, l_run, alpha, pf);
      if (any) scale_output<DH, QB, NW>(alpha, o);
      pv_block<DH, QB, NW>(stage(t), lane, pf, o);
    };
    int t = 0;
    for (; t + 2 < ntiles; t += 2) {
      step(t, scA, scB);
      step(t + 1, scB, scA);
    }
    if (t + 1 < ntiles) {
      step(t, scA, scB);
      finish(scB);
    } else {
      finish(scA);
    }
  } else {
  // full tiles: every kv of the tile lies below kv1
  for (int t = 0; t < ntiles - 1; ++t) {
    // tile t landed; the min(NS - 2, ntiles - 1 - t) tiles issued after it may be in flight
    const int younger = min(NS - 2, ntiles - 1 - t);
    if (NS >= 4 && younger >= 2) wait_copies_and_sync<2 * B::LOADS>();
    else if (NS >= 3 && younger >= 1) wait_copies_and_sync<B::LOADS>();
    else wait_copies_and_sync<0>();
    // stage (t + NS - 1) % NS was last read in iteration t - 1, which every wave has left
    if (t + NS - 1 < ntiles) issue(t + NS - 1);
    attn_tile<DH, QB, NW, false>(smem + (t % NS) * B::STAGE, kv0 + t * kKV, kv1, p.sl2, lane,
                                 qf, o, m_run, l_run);
  }
  {                                                         // the last tile
    const int t = ntiles - 1, t0 = kv0 + t * kKV;
    wait_copies_and_sync<0>();
    char* stage = smem + (t % NS) * B::STAGE;
    if (last_partial) {
      if (t0 + kKV > p.L) {
        zero_vt_tail<DH, NW>(stage, t0, p.L, tid);
        __syncthreads();
      }
      attn_tile<DH, QB, NW, true>(stage, t0, kv1, p.sl2, lane, qf, o, m_run, l_run);
    } else {
      attn_tile<DH, QB, NW, false>(stage, t0, kv1, p.sl2, lane, qf, o, m_run, l_run);
    }
  }
  }

  // O^T element i of block d: dh row d*32 + 8*(i/4) + 4h + i%4, query = this lane
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const float l_tot = halves_sum(l_run[qb]);
    const int rho = rho0 + qb * 32 + (lane & 31);
    if (rho >= M) continue;
    if (part) {
      const int64_t prow = (int64_t(split) * p.Hkv + g) * p.mcap + rho;
      uint16_t* op = p.opart + prow * DH;
      // bf16 partials: half the bytes written here and read by the merge
#pragma unroll
      for (int d = 0; d < B::DB; ++d)
#pragma unroll
        for (int i4 = 0; i4 < 4; ++i4)
          *reinterpret_cast<u32x2*>(op + d * 32 + 8 * i4 + 4 * h) =
              u32x2{cvt_bf16x2(o[qb][d][4 * i4], o[qb][d][4 * i4 + 1]),
                    cvt_bf16x2(o[qb][d][4 * i4 + 2], o[qb][d][4 * i4 + 3])};
      if (h == 0) { p.mlpart[prow * 2] = m_run[qb]; p.mlpart[prow * 2 + 1] = l_tot; }
    } else {
      const int r = rho / p.G, head = g * p.G + rho % p.G;
      char* O = reinterpret_cast<char*>(p.out + (int64_t(r) * p.Hq + head) * DH);
      const float inv = 1.f / l_tot;
#pragma unroll
      for (int d = 0; d < B::DB; ++d)
#pragma unroll
        for (int i4 = 0; i4 < 4; ++i4)
          *reinterpret_cast<u32x2*>(O + (d * 32 + 8 * i4 + 4 * h) * 2) =
              u32x2{cvt_bf16x2(o[qb][d][4 * i4] * inv, o[qb][d][4 * i4 + 1] * inv),
                    cvt_bf16x2(o[qb][d][4 * i4 + 2] * inv, o[qb][d][4 * i4 + 3] * inv)};
    }
  }
}

// log-sum-exp merge of the kv splits of the bf16 partial variant: one wave per
// packed query row.  Lane s holds split s's (m, l) (S <= 64), so the weights
// w_s = 2^(m_s - max m) and the denominator come from one round of loads and
// two wave reductions; the partial outputs are then summed with every lane
// owning DH / 64 (or one) consecutive elements, eight splits' loads in flight.
constexpr int kMaxSplits = 64;

template <int DH>
__global__ __launch_bounds__(256) void attn_bf16_merge_kernel(BP p, int QT, int grid) {
  constexpr int EPL = DH >= 64 ? DH / 64 : 1;              // elements per lane
  // (g, rho) over the plan's bound.  With p.spec the loads go out before the
  // row count arrives and rows past the count are dropped after it; without,
  // the count is read first (on a full step nothing is loaded).
  const int n_dev = *p.n_rows;
  const int row = blockIdx.x * 4 + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int g = row / p.mb, rho = row % p.mb;
  if (g >= p.Hkv) return;
  if (!p.spec) {
    const int n0 = min(n_dev, p.max_rows);
    if (n0 <= 0 || n0 > kPartialMaxRows || rho >= n0 * p.G) return;
  }
  const DPlan d{p.qa, p.S, p.per};
  const int lane = threadIdx.x & 63;
  const int64_t stride = int64_t(p.Hkv) * p.mcap;           // rows between consecutive splits
  const int64_t r0 = int64_t(g) * p.mcap + rho;
  float ms = -INFINITY, ls = 0.f;
  if (lane < d.S) {
    ms = p.mlpart[(lane * stride + r0) * 2];
    ls = p.mlpart[(lane * stride + r0) * 2 + 1];
  }
  const float mx = wave_max(ms);
  const float w = (ms == -INFINITY) ? 0.f : fast_exp2(ms - mx);
  const float den = wave_sum(w * ls);
  const int e0 = lane * EPL;
  const bool act = e0 < DH;
  float num[EPL];
#pragma unroll
  for (int k = 0; k < EPL; ++k) num[k] = 0.f;
  const uint16_t* op = p.opart + r0 * DH + (act ? e0 : 0);
  for (int s0 = 0; s0 < d.S; s0 += 8) {
    float v[8][EPL];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int s = min(s0 + u, d.S - 1);                  // clamped: weight 0 below
      const uint16_t* src = op + s * stride * DH;
      if constexpr (EPL == 2) {                            // two consecutive bf16: one 32-bit load
        const uint32_t w2 = *reinterpret_cast<const uint32_t*>(src);
        v[u][0] = bf16_lo(w2);
        v[u][1] = bf16_hi(w2);
      } else {
#pragma unroll
        for (int k = 0; k < EPL; ++k) v[u][k] = bf16_to_f32(src[k]);
      }
    }
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const float wu = (s0 + u < d.S) ? __int_as_float(__builtin_amdgcn_readlane(__float_as_int(w), s0 + u)) : 0.f;
#pragma unroll
      for (int k = 0; k < EPL; ++k) num[k] = fmaf(wu, v[u][k], num[k]);
    }
  }
  const int n = min(n_dev, p.max_rows);
  if (!act || n <= 0 || n > kPartialMaxRows || rho >= n * p.G) return;
  const int r = rho / p.G, head = g * p.G + rho % p.G;
  const float inv = 1.f / den;
#pragma unroll
  for (int k = 0; k < EPL; ++k)
    Elem<bf16_t>::store(p.out, (int64_t(r) * p.Hq + head) * DH + e0 + k, num[k] * inv);
}

// Launch shapes: waves per workgroup, 32-row query blocks per wave, LDS
// stages, and (partial variant) workgroups per CU in the grid.
struct BShape { int nw, qb, ns, wpc, pipe; };

// Measured on the Dream- and LLaDA-shaped workloads: eight waves of one query
// block, four stages and the pipelined schedule for head dims 64 / 128 (two
// waves per SIMD, next-tile QK under the current softmax); four waves for
// MHA partial steps (one query tile per head) and for head dim 32.
BShape partial_shape(int G, int dh) {
  if (dh == 32) return {4, G >= 2 ? 2 : 1, 3, 1, 0};
  return G >= 2 ? BShape{8, 1, 4, 1, 1} : BShape{4, 1, 3, 1, 0};
}
BShape full_shape(int dh) { return dh == 32 ? BShape{4, 2, 3, 1, 0} : BShape{8, 1, 4, 1, 1}; }

struct BPlan { int grid_p, mcap, smax; BShape sp; };

BPlan plan_bf16(int L, int Hkv, int G, int dh) {
  BPlan b;
  b.sp = partial_shape(G, dh);
  b.grid_p = (device_cu_count() * b.sp.wpc + 7) / 8 * 8;
  const int qt = b.sp.nw * 32 * b.sp.qb;
  b.mcap = (kPartialMaxRows * G + qt - 1) / qt * qt;
  const int tiles = (L + kKV - 1) / kKV;
  b.smax = max(1, min(min(b.grid_p / Hkv, kMaxSplits), (tiles + 1) / 2));
  return b;
}

size_t bf16_ws_bytes(int L, int Hkv, int G, int dh) {
  const BPlan b = plan_bf16(L, Hkv, G, dh);
  // bf16 partial O, then float (m, l)
  return size_t(b.smax) * Hkv * b.mcap * (size_t(dh) * 2 + 2 * sizeof(float));
}

template <int DH, int QB, int NW, int NS, bool PIPE>
hipError_t launch_bf16_kernel(const BP& p, unsigned grid, hipStream_t s) {
  const size_t lds = size_t(NS) * BG<DH, NW>::STAGE;
  hipLaunchKernelGGL((attn_bf16_kernel<DH, QB, NW, NS, PIPE>), dim3(grid), dim3(NW * 64), lds, s, p);
  return hipGetLastError();
}

// the shapes this library instantiates
template <int DH>
hipError_t launch_bf16_shape(const BP& p, BShape sh, unsigned grid, hipStream_t s) {
  if constexpr (DH >= 64) {
    if (sh.nw == 8 && sh.qb == 1 && sh.ns == 4 && sh.pipe) return launch_bf16_kernel<DH, 1, 8, 4, true>(p, grid, s);
  }
  if (sh.nw == 4 && sh.qb == 1 && sh.ns == 3 && !sh.pipe) return launch_bf16_kernel<DH, 1, 4, 3, false>(p, grid, s);
  if (sh.nw == 4 && sh.qb == 2 && sh.ns == 3 && !sh.pipe) return launch_bf16_kernel<DH, 2, 4, 3, false>(p, grid, s);
  return hipErrorInvalidValue;
}

template <int DH>
hipError_t launch_bf16(const AttnArgs& a, void* ws, hipStream_t s) {
  BP p;
  p.q = static_cast<const bf16_t*>(a.q); p.n_rows = a.n_rows_dev; p.max_rows = a.max_rows;
  p.kc = static_cast<const bf16_t*>(a.k_cache); p.vc = static_cast<const bf16_t*>(a.v_cache);
  p.L = a.L; p.L_cap = a.L_cap; p.Hq = a.Hq; p.Hkv = a.Hkv; p.G = a.Hq / a.Hkv;
  p.sl2 = a.scale * kLog2e; p.out = static_cast<bf16_t*>(a.out);
  const BPlan b = plan_bf16(a.L, a.Hkv, p.G, DH);
  if (ws == nullptr) return hipErrorInvalidValue;
  p.mcap = b.mcap; p.smax = b.smax;
  p.opart = static_cast<uint16_t*>(ws);
  p.mlpart = reinterpret_cast<float*>(p.opart + size_t(b.smax) * a.Hkv * b.mcap * DH);
  // split-KV variant (n <= 128): one workgroup per CU, then the merge.  The
  // plan is made here for the bound min(max_rows, 128) on the row count.
  const int bound = (a.small_rows > 0 && a.small_rows < a.max_rows) ? a.small_rows : a.max_rows;
  const int nb = bound < kPartialMaxRows ? bound : kPartialMaxRows;
  const DPlan d = split_plan(nb, p.G, b.sp.nw * 32 * b.sp.qb, a.Hkv, (a.L + kKV - 1) / kKV,
                             b.grid_p, b.smax);
  p.qa = d.qa; p.S = d.S; p.per = d.per; p.mb = nb * p.G;
  p.spec = (a.max_rows <= kPartialMaxRows || !(a.paths & kPathLarge)) ? 1 : 0;
  const bool small = (a.paths & kPathSmall) != 0;
  const bool large = a.max_rows > kPartialMaxRows && (a.paths & kPathLarge);
  // unsplit variant (n > 128); when the eight-wave query tiles would leave CUs
  // idle (e.g. MHA at L = 1024: 32 heads x 4 tiles), four-wave tiles of 128
  // rows double the workgroups
  BShape sh = full_shape(DH);
  unsigned grid_full = 0;
  if (large) {
    int qt = sh.nw * 32 * sh.qb;
    int64_t groups = (int64_t(a.max_rows) * p.G + qt - 1) / qt * a.Hkv;
    if (DH >= 64 && groups < device_cu_count()) {
      sh = BShape{4, 1, 3, 1, 0};
      qt = sh.nw * 32 * sh.qb;
      groups = (int64_t(a.max_rows) * p.G + qt - 1) / qt * a.Hkv;
    }
    grid_full = unsigned((groups + 7) / 8 * 8);
  }
  auto merge = [&]() {
    const int64_t rows = int64_t(a.Hkv) * p.mb;                     // (g, rho) rows of the bound
    hipLaunchKernelGGL((attn_bf16_merge_kernel<DH>), dim3(unsigned((rows + 3) / 4)), dim3(256), 0, s,
                       p, b.sp.nw * 32 * b.sp.qb, b.grid_p);
    return hipGetLastError();
  };
  // Both variants with one kernel shape and an unsplit grid no larger than
  // the split one (the LLaDA-shaped layer): one launch whose workgroups take
  // the split or the unsplit role from the device row count, saving the
  // launch of the variant that does not apply.  With a larger unsplit grid
  // (the Dream-shaped layer: 3592 workgroups at L = 32800) the workgroups
  // that exit at once on a partial step would queue behind the working ones
  // (one workgroup's LDS fills a CU) and cost far more than a launch.
  if (small && large && sh.nw == b.sp.nw && sh.qb == b.sp.qb && sh.ns == b.sp.ns &&
      sh.pipe == b.sp.pipe && grid_full <= unsigned(b.grid_p)) {
    p.partial = 2;
    const hipError_t e = launch_bf16_shape<DH>(p, sh, unsigned(b.grid_p), s);
    return e != hipSuccess ? e : merge();
  }
  if (small) {
    p.partial = 1;
    hipError_t e = launch_bf16_shape<DH>(p, b.sp, unsigned(b.grid_p), s);
    if (e == hipSuccess) e = merge();
    if (e != hipSuccess) return e;
  }
  if (!large) return hipSuccess;
  p.partial = 0;
  return launch_bf16_shape<DH>(p, sh, grid_full, s);
}

}  // namespace

size_t attn_ws_bytes(int max_rows, int L, int Hq, int Hkv, int dh) {
  (void)max_rows;
  // the larger of the two paths' needs (the dtype is not known here)
  const SplitPlan sp = plan_split(L, Hkv, Hq / Hkv);
  const size_t f32 = sp.S <= 1 ? 0 : size_t(sp.S) * Hkv * sp.mcap * (size_t(dh) + 2) * sizeof(float);
  const size_t b16 = bf16_ws_bytes(L, Hkv, Hq / Hkv, dh);
  return f32 > b16 ? f32 : b16;
}

hipError_t launch_attention(const AttnArgs& a, void* ws, hipStream_t s) {
  if (a.dtype == 1) {
    if (a.dh == 128) return launch_bf16<128>(a, ws, s);
    if (a.dh == 64) return launch_bf16<64>(a, ws, s);
    if (a.dh == 32) return launch_bf16<32>(a, ws, s);
  } else {
    if (a.dh == 128) return launch_typed<float, 128>(a, ws, s);
    if (a.dh == 64) return launch_typed<float, 64>(a, ws, s);
    if (a.dh == 32) return launch_typed<float, 32>(a, ws, s);
  }
  return hipErrorNotSupported;
}

}  // namespace ec
