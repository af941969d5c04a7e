// Launch description of decode attention over a compressed K/V cache.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace hq {

// queries per block: 4 (held in registers) for up to 4 queries per head,
// else 8 (read from LDS)
inline int attn_group(int64_t n_q) { return n_q <= 4 ? 4 : 8; }

struct AttnLaunch {
  const float* q;           // [n_heads][n_q][128]
  int64_t n_q;              // queries per head
  int64_t n_heads;
  const int8_t* k_idx;      // [n_heads][n_keys][128], E8 tile 128
  const uint32_t* k_coset;  // [n_keys]
  const float* k_scale;     // [n_keys]
  const int8_t* v_idx;
  const uint32_t* v_coset;
  const float* v_scale;
  int64_t n_keys;           // per head
  float* out;               // [n_heads][n_q][128]
  float* qr;                // workspace: the rotated, scaled queries
  float* part;              // workspace: per head, range and query m, l, acc[128]
  int64_t keys_per_wave;    // a range is four waves' keys
  int64_t n_ranges;         // per head
  uint32_t k_signs[4];
  uint32_t v_signs[4];
  int32_t k_dither, v_dither;
  uint32_t k_seed, v_seed;
  int64_t k_base, v_base;
  double q_scale;           // tau log2(e) / sqrt(128)
};

void attn_plan(int64_t n_heads, int64_t n_q, int64_t n_keys, int64_t& keys_per_wave,
               int64_t& n_ranges);
size_t attn_workspace(int64_t n_heads, int64_t n_q, int64_t n_keys);
// Blocks of the attention launch (ranges x query groups x heads).
int64_t attn_blocks(int64_t n_heads, int64_t n_q, int64_t n_keys);
hipError_t launch_attention(const AttnLaunch& a, hipStream_t s);

}  // namespace hq
