// Internal definitions shared by the host planner and the HIP launchers.
// Not part of the public ABI (include/kvq.h is).
#ifndef KVQ_INTERNAL_H_
#define KVQ_INTERNAL_H_

#include <stdint.h>

#include "../../include/kvq.h"

namespace kvq {

constexpr int kMaxLevels = 16;
constexpr int kLambdaGrid = 512;          // lambda grid points per octave
constexpr uint32_t kStateLow = 1u << 23;  // rANS normalisation bound L
constexpr int kRateFracBits = 16;

// Per-side (K or V) coding tables, host copy.  The decode-table entry packs
// f (bits 0-7), z - c (bits 8-15) and the symbol (bits 16-23): one lookup
// serves the state update and the level.
struct SideTables {
  int levels;
  int container_bytes;
  uint32_t freq[kMaxLevels];
  uint32_t cum[kMaxLevels];
  uint32_t rate_fx[kMaxLevels];
  // encoder division x / f as umulhi(x, rcp) >> shift (rcp == 0: x >> shift)
  uint32_t rcp[kMaxLevels];
  uint32_t rshift[kMaxLevels];
  uint32_t dec[256];
  uint32_t fp16_hi[kMaxLevels];  // high byte of fp16(v_m)
  uint32_t fp16_lo[kMaxLevels];  // low byte of fp16(v_m) (0 for integer levels <= 8)
  uint32_t fp16_bits[kMaxLevels];
  float level[kMaxLevels];       // v_m as stored (fp16), in grid units
  int affine;                    // v_m == m for every m
  uint32_t cheapest;   // lowest index with the smallest rate
  uint64_t budget_fx;  // (8C - 32) * 2^16
};

}  // namespace kvq

struct kvq_plan {
  kvq_params params;
  int n;                     // n_kv_heads * head_dim
  kvq::SideTables side[2];   // 0 = keys, 1 = values
  float lambda_grid[kvq::kLambdaGrid];
  float hadamard_scale;      // fp32(1 / sqrt(head_dim))
};

#endif  // KVQ_INTERNAL_H_
