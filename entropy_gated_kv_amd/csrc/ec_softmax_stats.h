// Online softmax statistics of a run of logits, shared by the entropy pass
// and the LM head's epilogue: for a run x with maximum m,
//   z = sum 2^u,  s2 = sum 2^u u,  u = (x - m) log2 e,
// give H = ln 2 (log2 z - s2 / z) and p1 = 1 / z (EntropyCache, Chinese
// summary page, section 2.2: the entropy of a decoded token's distribution).
// Two runs merge exactly by rescaling to the larger maximum.
#pragma once
#include <math.h>

#include "ec_device.h"
#include "ec_launch.h"

namespace ec {

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

__device__ __forceinline__ EntropyPartial empty_partial() {
  EntropyPartial p;
  p.m = -INFINITY; p.z = 0.f; p.s2 = 0.f; p.idx = kNoIdx;
  return p;
}

}  // namespace ec
