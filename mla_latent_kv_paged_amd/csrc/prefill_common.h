// Definitions shared by the chunked-prefill kernels (prefill.hip: expansion and the 16x16x32 attention;
// prefill_attn.hip: the 32x32x16 attention): the expanded K/V row layout, the LDS stage geometry of the
// attention rings, and small device helpers.
#pragma once
#include "mla_internal.h"

namespace mla {
namespace {

constexpr int kKV = DN + DR + DV;          // 320 values per expanded token row
constexpr int kKVBytes = kKV * 2;          // 640
constexpr int kGQ = kKV / 64;              // 5 granule groups (8 granules of 8 values) per token row
constexpr int kSubBytes = 16 * kKVBytes;   // a 16-token sub-block in LDS: 2 x 5 chunks of 1 KiB
constexpr int kPairBytes = 2 * kSubBytes;  // 32 tokens: one stage of the attention kernels' rings
constexpr float kMaxSlack = 8.f;           // lazy-rescale slack (log2 units), as in the decode

// chunk length of sequence b, clamped to the launch bound; 0 for an inconsistent prefix sum
__device__ __forceinline__ int chunk_of(const PrefillArgs& a, int b, int* first) {
  const int c0 = a.cu_q_lens[b];
  int n = a.cu_q_lens[b + 1] - c0;
  if (c0 < 0 || n < 0 || c0 > a.total_q || n > a.total_q - c0) n = 0;
  *first = c0;
  return n < a.max_q_len ? n : a.max_q_len;
}

// maxima without the canonicalising moves that fmaxf puts before each operand (the scores are
// MFMA results or -inf, never signalling NaNs)
__device__ __forceinline__ float vmax3(float x, float y, float z) {
  float r;
  asm("v_max3_f32 %0, %1, %2, %3" : "=v"(r) : "v"(x), "v"(y), "v"(z));
  return r;
}
__device__ __forceinline__ float vmax(float x, float y) {
  float r;
  asm("v_max_f32 %0, %1, %2" : "=v"(r) : "v"(x), "v"(y));
  return r;
}

// acc + the two bf16 halves of x, in fp32 (v_dot2c_f32_bf16 against (1, 1)): the row sums are
// taken over the same bf16 weights that the P.V MFMAs multiply
__device__ __forceinline__ float add_pk_bf16(uint32_t x, float acc) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, x), __builtin_bit_cast(bf16x2_t, 0x3f803f80u),
                                         acc, false);
}

}  // namespace
}  // namespace mla
