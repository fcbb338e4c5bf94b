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
// A workgroup (4 waves, 32 packed query rows each) owns one KV head, 128 packed
// rows and a range of kv.  Per 64-row kv tile (K and V^T tiles staged in LDS,
// double-buffered) each wave computes
//   S^T = K Q^T        (v_mfma_f32_32x32x16_bf16 / 32x32x2_f32; rows = kv)
// so a lane holds one query column and 32 kv scores: the running max and sum
// need only in-lane work plus one exchange with lane ^ 32.  K rows are loaded
// in a permuted order (bits 2 and 3 of the row index swapped) so that each
// lane's 16 accumulator values of a 32-row block are two runs of 8 consecutive
// kv; those runs are then directly the k-operand of
//   O^T += V^T P^T     (A = V^T tile rows from LDS, B = P^T from registers)
// with P rounded to the storage dtype (bf16 MFMA) or kept fp32.
// Two launches, each gated on the device row count: a split-KV variant for
// up to 128 selected rows (partial steps: enough kv splits to fill the chip,
// partial outputs merged by log-sum-exp in a second kernel) and an unsplit
// variant for more rows (full steps), which normalises and stores directly.
#include <math.h>

#include "ec_device.h"
#include "ec_launch.h"

namespace ec {

namespace {

constexpr int kThreads = 256;
constexpr int kKV = 64;              // kv rows per tile
constexpr int kQT = 128;             // packed query rows per workgroup
constexpr int kPartialMaxRows = 128; // rows handled by the split-KV variant

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
  {
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
  if (a.max_rows <= kPartialMaxRows) return hipSuccess;
  // unsplit variant (n > 128)
  p.S = 1; p.kv_per_split = (a.L + kKV - 1) / kKV * kKV; p.partial = 0;
  const int qtiles = (a.max_rows * p.G + kQT - 1) / kQT;
  hipLaunchKernelGGL((attn_kernel<T, DH>), dim3(unsigned(a.Hkv * qtiles)), dim3(kThreads), lds, s, p);
  return hipGetLastError();
}

}  // namespace

size_t attn_ws_bytes(int max_rows, int L, int Hq, int Hkv, int dh) {
  (void)max_rows;
  const SplitPlan sp = plan_split(L, Hkv, Hq / Hkv);
  if (sp.S <= 1) return 0;
  return size_t(sp.S) * Hkv * sp.mcap * (size_t(dh) + 2) * sizeof(float);
}

hipError_t launch_attention(const AttnArgs& a, void* ws, hipStream_t s) {
  if (a.dtype == 1) {
    if (a.dh == 128) return launch_typed<bf16_t, 128>(a, ws, s);
    if (a.dh == 64) return launch_typed<bf16_t, 64>(a, ws, s);
    if (a.dh == 32) return launch_typed<bf16_t, 32>(a, ws, s);
  } else {
    if (a.dh == 128) return launch_typed<float, 128>(a, ws, s);
    if (a.dh == 64) return launch_typed<float, 64>(a, ws, s);
    if (a.dh == 32) return launch_typed<float, 32>(a, ws, s);
  }
  return hipErrorNotSupported;
}

}  // namespace ec
