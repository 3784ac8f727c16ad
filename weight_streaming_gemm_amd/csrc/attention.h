// attention.h — arguments and launch of the decode attention (attention.hip),
// shared with the host library (not part of the C ABI).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stddef.h>

namespace qg {

// Decode attention of the agents' step rows (attention.hip).  q [A][rows][8 Hkv][128],
// caches [A][Hkv][cap][128] (bf16), lengths [A] (cached positions before the
// step's rows, clamped to [0, max_len]); partials per (agent, head, split).
constexpr int ATTN_HEAD_DIM = 128, ATTN_GROUP = 8, ATTN_MAX_ROWS = 4;
// Sequence splits: as many workgroups as stay resident in one round on an
// MI355X (256 CUs, one workgroup of the split kernel each: its registers leave
// room for one wave per SIMD), each split a multiple of the 32-position step.
constexpr int ATTN_RESIDENT = 256, ATTN_SPLIT_UNIT = 32;
struct AttnArgs {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  const int32_t* lengths;
  float* part_o;           // [A][Hkv][nsplit][32][128]
  float* part_ml;          // [A][Hkv][nsplit][32][2]: running max (base 2) and sum
  int32_t A, rows, Hkv, cap, max_len, nsplit;
  int32_t split;           // positions per split (a multiple of 32)
  float scale_log2;        // log2(e) / sqrt(128)
};
inline int attn_split_len(int A, int Hkv, int max_len, int rows) {
  const int64_t items = (int64_t)A * Hkv > 0 ? (int64_t)A * Hkv : 1;
  const int64_t target = ATTN_RESIDENT / items > 1 ? ATTN_RESIDENT / items : 1;   // splits per (agent, head)
  const int64_t total = (int64_t)max_len + rows;
  const int64_t per = (total + target - 1) / target;
  const int64_t split = (per + ATTN_SPLIT_UNIT - 1) / ATTN_SPLIT_UNIT * ATTN_SPLIT_UNIT;
  return (int)(split > ATTN_SPLIT_UNIT ? split : ATTN_SPLIT_UNIT);
}
inline int attn_splits(int A, int Hkv, int max_len, int rows) {
  const int split = attn_split_len(A, Hkv, max_len, rows);
  return (int)(((int64_t)max_len + rows + split - 1) / split);
}
inline size_t attn_ws_bytes(int A, int Hkv, int rows, int max_len) {
  return (size_t)A * Hkv * attn_splits(A, Hkv, max_len, rows) * 32 * (ATTN_HEAD_DIM + 2) * 4;
}
hipError_t launch_attention(const AttnArgs& a, float* out, hipStream_t st);

}  // namespace qg
