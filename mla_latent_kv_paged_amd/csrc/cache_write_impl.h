// Device code of the latent cache write, shared by the cache-write kernels and the decode step's
// first launch (which runs these tokens beside the query absorption).  What is computed: see
// cache_write.hip.
#pragma once
#include "mla_internal.h"

namespace mla {

__device__ __forceinline__ double load_f64(const uint16_t* p, int64_t i) { return double(bf16_to_f32(p[i])); }
__device__ __forceinline__ double load_f64(const float* p, int64_t i) { return double(p[i]); }
__device__ __forceinline__ void store_round(uint16_t* p, int64_t i, double v) { p[i] = f64_to_bf16(v); }
__device__ __forceinline__ void store_round(float* p, int64_t i, double v) { p[i] = float(v); }

// token j of a cache write, by one wavefront (lane = lane id): inputs of type Tin (the storage
// dtype, or fp32 rows of the layer step's projection), cache rows of type T
template <typename T, typename Tin = T>
__device__ __forceinline__ void cache_write_token(const CacheWriteArgs& a, int j, int lane) {
#pragma clang fp contract(off)
  if (j >= a.T) return;
  // every load of the token is issued before any of them is inspected (one memory round trip)
  const Tin* c = static_cast<const Tin*>(a.c_kv) + int64_t(j) * a.c_stride;
  const Tin* k = static_cast<const Tin*>(a.k_pe) + int64_t(j) * a.k_stride;
  const int slot = a.slots[j];
  const int pos = a.positions[j];
  double x[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) x[e] = load_f64(c, lane * 8 + e);
  const double kx0 = load_f64(k, 2 * (lane & (NPAIR - 1)));
  const double kx1 = load_f64(k, 2 * (lane & (NPAIR - 1)) + 1);
  double gm[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) gm[e] = a.gamma[lane * 8 + e];
  if (slot < 0 || int64_t(slot) >= a.num_slots) return;  // padding or out-of-pool slot: skipped
  T* dst = static_cast<T*>(a.cache) + int64_t(slot) * ROW;
  const bool pos_ok = pos >= 0 && pos <= a.max_position;
  const double2 cs = a.rope[int64_t(pos_ok ? pos : 0) * NPAIR + (lane & (NPAIR - 1))];

  // RMSNorm over the 512 latent channels (fp64): x / sqrt(mean(x^2) + eps) * gamma
  double ss = 0.0;
#pragma unroll
  for (int e = 0; e < 8; ++e) ss += x[e] * x[e];
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) ss += __shfl_xor(ss, off, 64);
  const double denom = sqrt(ss / double(DC) + a.eps);
  const double nan = __builtin_nan("");
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const double y = x[e] / denom * gm[e];
    store_round(dst, lane * 8 + e, pos_ok ? y : nan);
  }

  // RoPE on k_pe: pair i = (x[2i], x[2i+1]) rotated by pos * theta^(-2i/64)
  if (lane < NPAIR) {
    const double x0 = kx0, x1 = kx1;
    double y0 = nan, y1 = nan;
    if (pos_ok) {
      y0 = x0 * cs.x - x1 * cs.y;
      y1 = x0 * cs.y + x1 * cs.x;
    }
    store_round(dst, DC + 2 * lane, y0);
    store_round(dst, DC + 2 * lane + 1, y1);
  }
}

// FP8 E4M3 code of x (|x| <= 448): nearest value, ties to the even code.  Below the smallest normal
// 2^-6 the values are the multiples of 2^-9 (code = the multiple; 8 lands on the smallest normal);
// above, x = (1 + m/8) 2^e with code (e + 7) << 3 | m, a rounding carry moving to the next binade.
// Every step is exact in fp64 except the one rint, which rounds half to even.
__device__ __forceinline__ uint32_t e4m3_code(double x) {
  const double ax = fabs(x);
  uint32_t code;
  if (ax < 0.015625) {
    code = uint32_t(rint(ax * 512.0));
  } else {
    int E;
    const double f = frexp(ax, &E);  // ax = f 2^E, f in [0.5, 1)
    int e = E - 1;
    double mant = rint((2.0 * f - 1.0) * 8.0);
    if (mant == 8.0) {
      mant = 0.0;
      ++e;
    }
    code = (uint32_t(e + 7) << 3) | uint32_t(mant);
  }
  return (x < 0.0 && code != 0) ? (code | 0x80u) : code;
}

// S1 with FP8 latent rows (row layout in mla_internal.h): as cache_write_kernel up to the fp64
// normed latent y and the rotated rope pair; then per group of 128 channels (16 lanes) the scale
// s = fp32(amax / 448), stepped up one fp32 value if amax / s would exceed 448 (1 for an all-zero
// group), and codes e4m3(y / s) with the quotient in fp64.  The rope values are rounded to bf16.
// Inputs of type Tin: bf16, or fp32 rows of the layer step's projection.
template <typename Tin = uint16_t>
__device__ __forceinline__ void cache_write_fp8_token(const CacheWriteArgs& a, int j, int lane) {
#pragma clang fp contract(off)
  if (j >= a.T) return;
  const Tin* c = static_cast<const Tin*>(a.c_kv) + int64_t(j) * a.c_stride;
  const Tin* k = static_cast<const Tin*>(a.k_pe) + int64_t(j) * a.k_stride;
  const int slot = a.slots[j];
  const int pos = a.positions[j];
  double x[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) x[e] = load_f64(c, lane * 8 + e);
  const double kx0 = load_f64(k, 2 * (lane & (NPAIR - 1)));
  const double kx1 = load_f64(k, 2 * (lane & (NPAIR - 1)) + 1);
  double gm[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) gm[e] = a.gamma[lane * 8 + e];
  if (slot < 0 || int64_t(slot) >= a.num_slots) return;
  uint8_t* dst = static_cast<uint8_t*>(a.cache) + int64_t(slot) * kFp8Row;
  const bool pos_ok = pos >= 0 && pos <= a.max_position;
  const double2 cs = a.rope[int64_t(pos_ok ? pos : 0) * NPAIR + (lane & (NPAIR - 1))];

  double ss = 0.0;
#pragma unroll
  for (int e = 0; e < 8; ++e) ss += x[e] * x[e];
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) ss += __shfl_xor(ss, off, 64);
  const double denom = sqrt(ss / double(DC) + a.eps);
  double y[8];
  double amax = 0.0;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    y[e] = x[e] / denom * gm[e];
    amax = fmax(amax, fabs(y[e]));
  }
#pragma unroll
  for (int off = 8; off >= 1; off >>= 1) amax = fmax(amax, __shfl_xor(amax, off, 64));  // 16-lane groups
  float s = 1.f;
  if (amax > 0.0) {
    s = float(amax / 448.0);
    if (amax > 448.0 * double(s)) s = __uint_as_float(__float_as_uint(s) + 1u);
  }
  uint32_t lo = 0, hi = 0;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    lo |= e4m3_code(y[e] / double(s)) << (8 * e);
    hi |= e4m3_code(y[e + 4] / double(s)) << (8 * e);
  }
  if (!pos_ok) lo = hi = 0x7f7f7f7fu;  // NaN codes: the error stays visible downstream
  *reinterpret_cast<u32x2_t*>(dst + 8 * lane) = u32x2_t{lo, hi};
  if (lane < NPAIR) {
    double y0 = __builtin_nan(""), y1 = __builtin_nan("");
    if (pos_ok) {
      y0 = kx0 * cs.x - kx1 * cs.y;
      y1 = kx0 * cs.y + kx1 * cs.x;
    }
    *reinterpret_cast<uint32_t*>(dst + DC + 4 * lane) = uint32_t(f64_to_bf16(y0)) | (uint32_t(f64_to_bf16(y1)) << 16);
  }
  if ((lane & 15) == 0) *reinterpret_cast<float*>(dst + DC + 2 * DR + 4 * (lane >> 4)) = pos_ok ? s : __builtin_nanf("");
}

}  // namespace mla
