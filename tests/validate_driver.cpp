// Host-only driver of the C ABI's argument checks (ec_validate.cpp), built by
// tests/test_abi.py with the host compiler's address and undefined-behaviour
// sanitizers.  It checks the documented status of hand-made cases, then calls
// every check with seeded random arguments, extreme integers included, so the
// sanitizers see the checks' arithmetic and pointer reads over a wide range.
// Pointer arguments are either NULL or the addresses of host buffers; nothing
// is dereferenced except what the checks themselves read (the model's layer
// array and the state's cache arrays, sized as the ABI requires).
// Exit status 0: every expectation held.
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include <random>
#include <vector>

#include "ec_validate.h"

namespace {

int failures = 0;
#define EXPECT(cond)                                                        \
  do {                                                                      \
    if (!(cond)) {                                                          \
      ++failures;                                                           \
      fprintf(stderr, "%s:%d: expectation failed: %s\n", __FILE__, __LINE__, #cond); \
    }                                                                       \
  } while (0)

alignas(16) unsigned char buf[4096];
void* A = buf + 16;        // aligned
void* U = buf + 20;        // misaligned

std::mt19937_64 rng(12345);

int64_t pick64() {
  static const int64_t special[] = {INT64_MIN, INT64_MIN + 1, -1, 0, 1, 2, 15, 16, 17, 64, 127,
                                    128, 1024, 126464, 152064, (int64_t(1) << 24),
                                    (int64_t(1) << 30), (int64_t(1) << 31), INT32_MAX,
                                    int64_t(INT32_MAX) + 1, INT64_MAX - 1, INT64_MAX};
  if (rng() % 2) return special[rng() % (sizeof(special) / sizeof(special[0]))];
  return int64_t(rng());
}
int32_t pick32() {
  static const int32_t special[] = {INT32_MIN, INT32_MIN + 1, -2, -1, 0, 1, 2, 3, 4, 7, 16, 28,
                                    32, 64, 96, 128, 129, 1024, 1025, 4096, 32800, 262144,
                                    262145, INT32_MAX - 1, INT32_MAX};
  if (rng() % 2) return special[rng() % (sizeof(special) / sizeof(special[0]))];
  return int32_t(uint32_t(rng()));
}
template <typename T> T* ptr() {
  const int c = int(rng() % 4);
  return c == 0 ? nullptr : static_cast<T*>(c == 1 ? U : A);
}
float pickf() {
  static const float special[] = {-1.f, 0.f, 1e-30f, 0.088388f, 1.f, 1e30f};
  const int c = int(rng() % 8);
  if (c == 6) return __builtin_inff();
  if (c == 7) return __builtin_nanf("");
  return special[c];
}

void hand_cases() {
  float f[4];
  int32_t i[4];
  // entropy
  EXPECT(ec::check_entropy(A, EC_BF16, 4, 100, 104, nullptr, nullptr, 0, f, f, i) == EC_OK);
  EXPECT(ec::check_entropy(nullptr, EC_BF16, 4, 100, 104, nullptr, nullptr, 0, f, f, i) == EC_E_NULL);
  EXPECT(ec::check_entropy(A, 7, 4, 100, 104, nullptr, nullptr, 0, f, f, i) == EC_E_DTYPE);
  EXPECT(ec::check_entropy(A, EC_BF16, 4, 100, 99, nullptr, nullptr, 0, f, f, i) == EC_E_SHAPE);
  EXPECT(ec::check_entropy(A, EC_BF16, 4, 100, 101, nullptr, nullptr, 0, f, f, i) == EC_E_ALIGN);
  EXPECT(ec::check_entropy(U, EC_BF16, 4, 100, 104, nullptr, nullptr, 0, f, f, i) == EC_E_ALIGN);
  EXPECT(ec::check_entropy(A, EC_BF16, 4, 100, INT64_MAX, nullptr, nullptr, 0, f, f, i) == EC_E_UNSUPPORTED);
  EXPECT(ec::check_entropy(A, EC_BF16, 4, 100, 104, i, nullptr, 4, f, f, i) == EC_E_NULL);
  // packed LM head
  EXPECT(ec::check_pack(A, 1024, 256, EC_BF16, buf + 2048) == EC_E_SHAPE);   // overlaps its source
  EXPECT(ec::check_pack(buf, 16, 32, EC_BF16, buf + 1024) == EC_OK);
  EXPECT(ec::check_pack(nullptr, 16, 32, EC_BF16, buf + 1024) == EC_E_NULL);
  EXPECT(ec::check_pack(buf, 16, 32, EC_F32, buf + 1024) == EC_E_DTYPE);
  EXPECT(ec::check_pack(buf, 24, 32, EC_BF16, buf + 1024) == EC_E_SHAPE);
  EXPECT(ec::check_pack(buf, 16, 32, EC_BF16, U) == EC_E_ALIGN);
  EXPECT(ec::check_pack(buf, INT32_MAX - 15, INT32_MAX - 31, EC_BF16, buf + 1024) == EC_E_UNSUPPORTED);
  // selection
  EXPECT(ec::check_select(i, reinterpret_cast<uint8_t*>(A), 10, 0, 4, 0, i, i, 16, 4, i, i) == EC_OK);
  EXPECT(ec::check_select(i, reinterpret_cast<uint8_t*>(A), 10, 0, 4, 1, i, i, 16, 4, i, i) == EC_OK);
  EXPECT(ec::check_select(i, reinterpret_cast<uint8_t*>(A), 10, 8, 4, 0, i, i, 16, 4, i, i) == EC_E_SHAPE);
  EXPECT(ec::check_select(i, reinterpret_cast<uint8_t*>(A), 10, INT32_MAX, 4, 0, i, i, 16, 4, i, i) == EC_E_SHAPE);
  EXPECT(ec::check_select(i, reinterpret_cast<uint8_t*>(A), 262145, 0, 4, 0, i, i, 16, 4, i, i) == EC_E_UNSUPPORTED);
  EXPECT(ec::check_select(i, reinterpret_cast<uint8_t*>(A), 10, -1, 4, 1, i, i, 16, 4, i, i) == EC_E_SHAPE);
  EXPECT(ec::check_select(i, reinterpret_cast<uint8_t*>(A), 10, 0, 4, 2, i, i, 16, 4, i, i) == EC_E_SHAPE);
  // refresh and attention
  EXPECT(ec::check_refresh(A, 4096, i, i, 96, A, 4096, 32, 32, 128, EC_BF16, A, A, A, 1024, nullptr) == EC_OK);
  EXPECT(ec::check_refresh(A, 4096, i, i, 96, A, 4096, 32, 32, 48, EC_BF16, A, A, A, 1024, nullptr) == EC_E_UNSUPPORTED);
  EXPECT(ec::check_refresh(A, 4096, i, i, 96, A, 4096, INT32_MIN, -1, 128, EC_BF16, A, A, A, 1024, nullptr) == EC_E_SHAPE);
  EXPECT(ec::check_attention(A, i, 96, A, A, 8224, 8224, 28, 4, 128, 0.088f, EC_BF16, A, A) == EC_OK);
  EXPECT(ec::check_attention(A, i, 96, A, A, 8225, 8224, 28, 4, 128, 0.088f, EC_BF16, A, A) == EC_E_SHAPE);
  EXPECT(ec::check_attention(A, i, 96, A, A, 8224, 8224, 28, 4, 128, __builtin_nanf(""), EC_BF16, A, A) == EC_E_SHAPE);
  EXPECT(ec::check_attention(A, i, 96, A, A, 8224, 8224, 68, 4, 128, 0.088f, EC_BF16, A, A) == EC_E_UNSUPPORTED);
  EXPECT(ec::check_attention(A, i, 96, A, A, 8224, 8224, 28, 4, 128, 0.088f, EC_BF16, A, U) == EC_E_ALIGN);
}

// A model and state with every pointer valid (aligned host addresses).
struct StepCase {
  std::vector<ec_layer> layers;
  std::vector<void*> kc, vc;
  ec_model m{};
  ec_state st{};
  ec_step_cfg c{};
  explicit StepCase(int n_layers) : layers(size_t(n_layers)), kc(size_t(n_layers), A),
                                    vc(size_t(n_layers), A) {
    for (auto& l : layers) l = ec_layer{A, A, A, A, A, A, A};
    m.n_layers = n_layers; m.d = 256; m.Hq = 4; m.Hkv = 2; m.dh = 64; m.d_ffn = 512;
    m.V = 2048; m.L_cap = 256; m.dtype = EC_BF16; m.rms_eps = 1e-5f;
    m.tok_emb = A; m.pos_emb = A; m.layers = layers.data(); m.norm_final = A; m.w_lm = A;
    m.logit_scale = nullptr;
    st.L = 160; st.tokens = static_cast<int32_t*>(A); st.is_masked = static_cast<uint8_t*>(A);
    st.history = static_cast<int32_t*>(A); st.history_len = static_cast<int32_t*>(A);
    st.history_cap = 64; st.full_flag = static_cast<int32_t*>(A); st.k_cache = kc.data();
    st.v_cache = vc.data(); st.rows = static_cast<int32_t*>(A); st.n_rows = static_cast<int32_t*>(A);
    st.logits = A; st.row_entropy = static_cast<float*>(A); st.row_argmax = static_cast<int32_t*>(A);
    st.row_top1 = static_cast<float*>(A); st.chosen = static_cast<int32_t*>(A);
    st.n_chosen = static_cast<int32_t*>(A); st.e_max = static_cast<float*>(A);
    st.kv_drift = nullptr; st.attn_out = nullptr;
    c.tau = 1.f; c.k = 16; c.n_unmask = 2; c.block_start = 96; c.block_len = 32;
    c.mode = EC_MODE_DEVICE; c.block_causal = 0;
  }
};

void step_cases() {
  {
    StepCase s(2);
    EXPECT(ec::check_step(&s.m, &s.st, &s.c, A) == EC_OK);
    EXPECT(ec::check_step(&s.m, &s.st, &s.c, nullptr) == EC_E_NULL);
    EXPECT(ec::check_step(&s.m, &s.st, &s.c, U) == EC_E_ALIGN);
    s.st.attn_out = U;
    EXPECT(ec::check_step(&s.m, &s.st, &s.c, A) == EC_E_ALIGN);
    s.st.attn_out = nullptr;
    s.layers[1].w_down = nullptr;
    EXPECT(ec::check_step(&s.m, &s.st, &s.c, A) == EC_E_NULL);
  }
  {
    StepCase s(1);
    s.c.block_start = INT32_MAX;                       // block_start + block_len must not wrap
    EXPECT(ec::check_step(&s.m, &s.st, &s.c, A) == EC_E_SHAPE);
    s.c.block_start = 96;
    s.m.Hq = INT32_MAX; s.m.Hkv = 1; s.m.dh = 128;     // Hq * dh must not wrap
    EXPECT(ec::check_step(&s.m, &s.st, &s.c, A) == EC_E_UNSUPPORTED);
  }
  {
    StepCase s(1);
    s.m.V = 2064;                                      // not whole 32-column blocks
    EXPECT(ec::check_step(&s.m, &s.st, &s.c, A) == EC_E_UNSUPPORTED);
    s.m.w_lm = nullptr;                                // no LM head: the caller decodes
    EXPECT(ec::check_step(&s.m, &s.st, &s.c, A) == EC_OK);
  }
  {
    StepCase s(1);                                     // no logits buffer
    s.st.logits = nullptr;
    EXPECT(ec::check_step(&s.m, &s.st, &s.c, A) == EC_E_NULL);        // no packed copy
    s.m.w_lm_packed = A;
    EXPECT(ec::check_step(&s.m, &s.st, &s.c, A) == EC_E_UNSUPPORTED); // V = 2048: 32 column tiles
    s.m.V = 32768;
    EXPECT(ec::check_step(&s.m, &s.st, &s.c, A) == EC_OK);
    s.m.d = 384;                                       // d % 256 != 0
    EXPECT(ec::check_step(&s.m, &s.st, &s.c, A) == EC_E_UNSUPPORTED);
    s.m.d = 256;
    s.c.block_len = 33;
    EXPECT(ec::check_step(&s.m, &s.st, &s.c, A) == EC_E_UNSUPPORTED);
  }
}

void fuzz(int rounds) {
  int32_t iv[64];
  float fv[64];
  for (int r = 0; r < rounds; ++r) {
    (void)ec::check_entropy(ptr<void>(), pick32() % 3, pick64(), pick64(), pick64(),
                            ptr<int32_t>(), ptr<int32_t>(), pick32(), ptr<float>(), ptr<float>(),
                            ptr<int32_t>());
    (void)ec::check_pack(ptr<void>(), pick32(), pick32(), pick32() % 3, ptr<void>());
    (void)ec::check_select(ptr<int32_t>(), ptr<uint8_t>(), pick32(), pick32(), pick32(), pick32() % 3,
                           ptr<int32_t>(), ptr<int32_t>(), pick32(), pick32(), ptr<int32_t>(),
                           ptr<int32_t>());
    (void)ec::check_refresh(ptr<void>(), pick64(), ptr<int32_t>(), ptr<int32_t>(), pick32(),
                            ptr<void>(), pick32(), pick32(), pick32(), pick32(), pick32() % 3,
                            ptr<void>(), ptr<void>(), ptr<void>(), pick32(), ptr<void>());
    (void)ec::check_attention(ptr<void>(), ptr<int32_t>(), pick32(), ptr<void>(), ptr<void>(),
                              pick32(), pick32(), pick32(), pick32(), pick32(), pickf(),
                              pick32() % 3, ptr<void>(), ptr<void>());
    // a step: the layer and cache arrays hold n_layers entries, as the ABI requires
    const int n_layers = 1 + int(rng() % 4);
    StepCase s(n_layers);
    s.m.d = pick32(); s.m.Hq = pick32(); s.m.Hkv = pick32(); s.m.dh = pick32();
    s.m.d_ffn = pick32(); s.m.V = pick32(); s.m.L_cap = pick32(); s.m.dtype = pick32() % 3;
    if (rng() % 2) s.m.w_lm = nullptr;
    if (rng() % 4 == 0) s.m.norm_final = ptr<void>();
    s.st.L = pick32(); s.st.history_cap = pick32();
    s.c.k = pick32(); s.c.n_unmask = pick32(); s.c.block_start = pick32();
    s.c.block_len = pick32(); s.c.mode = pick32() % 4; s.c.block_causal = pick32() % 3;
    if (rng() % 4 == 0) s.st.attn_out = ptr<void>();
    if (rng() % 4 == 0) s.m.w_lm_packed = ptr<void>();
    if (rng() % 4 == 0) s.layers[rng() % size_t(n_layers)].w_o = ptr<void>();
    if (rng() % 4 == 0) s.kc[rng() % size_t(n_layers)] = ptr<void>();
    (void)ec::check_step(&s.m, &s.st, &s.c, ptr<void>());
    (void)ec::model_ok(&s.m);
  }
  (void)iv;
  (void)fv;
}

}  // namespace

int main() {
  hand_cases();
  step_cases();
  fuzz(200000);
  if (failures) {
    fprintf(stderr, "%d expectation(s) failed\n", failures);
    return 1;
  }
  printf("validation checks: all expectations held, fuzz done\n");
  return 0;
}
