// Size limits shared by the host-side argument checks (ec_validate.cpp, which
// builds without HIP) and the kernels that rely on them.
#pragma once
#include <stdint.h>

namespace ec {

// Device row counts up to this run the small-row kernels (skinny GEMM,
// split-KV attention); larger counts run the tiled GEMM and unsplit attention.
constexpr int kSmallMaxRows = 128;
// Longest sequence the row selection handles (its LDS bitmap is L / 8 bytes).
constexpr int32_t kSelectMaxL = 262144;
// Most rows one step decodes from (the block length): one workgroup folds them.
constexpr int32_t kStepMaxRows = 1024;
// Reduction dimensions of the GEMMs (d, Hq * dh, d_ffn) are multiples of the
// k one skinny iteration covers: 128 for bf16, 64 for fp32.
constexpr int kKMultipleBf16 = 128;
constexpr int kKMultipleF32 = 64;
inline int k_multiple(int32_t dtype) { return dtype == 1 ? kKMultipleBf16 : kKMultipleF32; }
// Supported head dimensions and query heads per KV head.
inline bool head_dim_ok(int32_t dh) { return dh == 32 || dh == 64 || dh == 128; }
constexpr int kMaxGroup = 16;
// The packed LM-head kernel runs for at most kLmStatRows rows, at least
// kLmMinTiles column tiles of 64 and d a multiple of its k-block; only that
// kernel can write a step's softmax statistics in place of its logits.
constexpr int32_t kLmStatRows = 32;
constexpr int32_t kLmMinTiles = 512;
constexpr int32_t kLmKBlock = 256;

}  // namespace ec
