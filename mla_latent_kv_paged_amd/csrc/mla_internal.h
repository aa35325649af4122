// Internal declarations shared by the host API and the kernels of libmla (gfx950 only).
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "mla.h"

namespace mla {

// ------------------------------------------------------------------------------------ launches

// Timing of the kernels of one profiled region (mla_profile_enable).  While set, launch() hands the
// region's events to the dispatch itself (hipExtLaunchKernelGGL): the first launch's start and each
// launch's end.  The elapsed time is then the span of the kernels' own execution, without the queue's
// time between a marker and the dispatch that follows it.
struct LaunchEvents {
  hipEvent_t start;
  hipEvent_t stop;
  bool started;
};
extern thread_local LaunchEvents* t_launch_events;

// Every kernel of the library is launched through here (the arguments are converted to the
// kernel's parameter types, as a triple-chevron launch does).
template <typename... P>
inline void launch(void (*kernel)(P...), dim3 grid, dim3 block, uint32_t shmem, hipStream_t s,
                   typename std::common_type<P>::type... args) {
  LaunchEvents* e = t_launch_events;
  if (e == nullptr) {
    kernel<<<grid, block, shmem, s>>>(args...);
    return;
  }
  hipExtLaunchKernelGGL(kernel, grid, block, shmem, s, e->started ? nullptr : e->start, e->stop, 0u, args...);
  e->started = true;
}

// Fixed MLA dimensions (DeepSeek-V2 / V2-Lite shapes).
constexpr int DC = 512;        // kv_lora_rank: latent width
constexpr int DR = 64;         // qk_rope_head_dim: decoupled-RoPE key width
constexpr int DN = 128;        // qk_nope_head_dim
constexpr int DV = 128;        // v_head_dim
constexpr int ROW = DC + DR;   // 576 values per cache slot
constexpr int QW = DN + DR;    // 192 values per head of q
constexpr int BLK = 16;        // tokens per paged block
constexpr int NPAIR = DR / 2;  // RoPE pairs
// FP8 cache rows: [DC e4m3 codes | DR bf16 rope values | 4 fp32 group scales (128 channels each)]
constexpr int kFp8Row = DC + 2 * DR + 16;  // 656 bytes
constexpr int kFp8Block = BLK * kFp8Row;   // 10,496 bytes

// ------------------------------------------------------------------------------ kernel arguments

struct AbsorbArgs {
  const void* kv_b_proj;  // [H*(DN+DV), DC]
  void* W_uk;             // [H, DN, DC]  (fp32 query kernel)
  void* W_ukT;            // [H, DC, DN]  (MFMA query kernel: K = DN contiguous)
  void* W_uv;             // [H, DV, DC]  (MFMA output kernel: K = DC contiguous)
  void* W_uvT;            // [H, DC, DV]  (fp32 output kernel)
  int32_t H;
};

struct CacheWriteArgs {
  const void* c_kv;
  int64_t c_stride;  // elements
  const void* k_pe;
  int64_t k_stride;  // elements
  const int32_t* positions;
  const int32_t* slots;
  int32_t T;
  void* cache;
  int64_t num_slots;     // num_blocks * BLK
  const double* gamma;   // [DC]
  const double2* rope;   // [(max_position+1) * NPAIR] (cos, sin)
  int32_t max_position;
  double eps;
  int32_t in_f32;        // 1: c_kv / k_pe are fp32 rows (the layer step's projection), else the storage dtype
};

struct QAbsorbArgs {
  const void* q;          // [n_q, H, QW]
  const void* W_uk;       // [H, DN, DC]
  const void* W_ukT;      // [H, DC, DN]
  const double2* rope;
  const int32_t* seq_lens;
  int32_t q_len;
  int32_t n_q;
  int32_t H;
  int32_t max_seq_len;
  int32_t max_position;
  float qscale;           // softmax_scale * log2(e): scores come out in log2 units
  void* qcat;             // [n_q, H, ROW] (storage dtype): [q_lat | q_pe'] * qscale
};

struct DecodeArgs {
  int32_t batch;
  const void* cache;
  const void* zero_block;  // BLK * ROW zero values of the storage dtype (read by masked lanes)
  int32_t num_blocks;
  const int32_t* block_table;
  int32_t bt_stride;
  const int32_t* seq_lens;
  int32_t max_seq_len;
  int32_t q_len;
  int32_t H;
  const void* qcat;
  float* part_acc;        // fp32 kernel: [n_q*H*n_split, DC] unnormalised accumulators
  uint16_t* part_o16;     // bf16 kernels (same memory): [rows, DC] fp16 o = acc / l (0 when l = 0)
  float2* part_ml;        // [rows] (running max in log2 units, sum); (-inf, 0): nothing visible
  float* part_scale;      // bf16 kernels: [rows] the power of two the fp16 row was divided by
  int32_t split_blocks;
  int32_t n_split;
  int32_t n_rt;           // row tiles per sequence: of 16 rows ((H/16) * q_len), or of 32 for the 32-row kernel
  int32_t units;          // batch * n_split * n_rt work items; the 32-row kernel: its workgroup count
  int2* piece_tbl;        // 32-row kernel: per stream (first piece id, piece count), written by workgroup 0
};

// Chunked prefill (mla_prefill).  Sequence b owns query rows cu_q_lens[b] .. cu_q_lens[b+1]-1 at
// positions ctx_b - n_b .. ctx_b - 1.  Workspace: kv [batch, H, t_pad, DN + DR + DV] expanded
// token rows [K_nope | k_pe | V] per (sequence, head).
// tokens per expansion workgroup; the workspace's rows per (sequence, head) are a multiple of it
constexpr int kPrefillTokens = 1024;

struct PrefillArgs {
  int32_t batch;
  int32_t H;
  const void* q;               // [total_q, H, DN + DR] bf16, un-rotated
  const int32_t* cu_q_lens;    // [batch + 1]
  int32_t total_q;
  int32_t max_q_len;           // an upper bound of every chunk length (sizes the grids)
  const void* cache;           // bf16 [num_blocks, BLK, 1, ROW], or FP8 rows [num_blocks, BLK, 1, kFp8Row]
  const void* zero_block;
  int32_t num_blocks;
  const int32_t* block_table;
  int32_t bt_stride;
  const int32_t* seq_lens;
  int32_t max_seq_len;
  int32_t max_position;
  int32_t t_pad;               // token rows per (sequence, head) in kv: max_seq_len rounded up to kPrefillTokens
  const double2* rope;
  float qscale;                // softmax scale * log2(e)
  const uint16_t* W_uk;        // [H, DN, DC]
  const uint16_t* W_uv;        // [H, DV, DC]
  uint16_t* kv;
  uint16_t* qpe;               // [total_q, H, DR] bf16: RoPE(q_pe) at the rows' positions (written by the prep)
  uint16_t* lat;               // FP8 cache: [batch, t_pad, ROW] bf16 rows dequantised from it (else null)
  void* out;                   // [total_q, H, DV] bf16
  int32_t units;               // work items of the kernel being launched
};

struct CombineArgs {
  const float* part_acc;  // fp32 path
  const uint16_t* part_o16;  // bf16 path: fp16 normalised partials (acc / l)
  const float2* part_ml;
  const float* part_scale;  // bf16 path: the fp16 partial row times this is o
  const int32_t* seq_lens;
  int32_t max_seq_len;
  int32_t q_len;
  int32_t n_q;
  int32_t H;
  int32_t split_blocks;
  int32_t n_split;
  const void* W_uv;       // [H, DV, DC]
  const void* W_uvT;      // [H, DC, DV]
  void* out;              // [n_q, H, DV]
  // partials by piece (32-row kernel) instead of by split: row (n, h) of sequence b = n / q_len has
  // rr = (n % q_len) H + h, stream s = b n_grp + rr / rows_per_piece; piece k of s is partial
  // (piece_tbl[s].x + k) rows_per_piece + rr % rows_per_piece, k < piece_tbl[s].y
  const int2* piece_tbl;  // null: by split
  int32_t rows_per_piece;
  int32_t n_grp;
  int32_t v_parts;        // bf16: output channels split over this many workgroups (1 or 4)
  int32_t rows_wg;        // bf16: query rows per workgroup, 16 (combine_bf16_kernel) or 64 (combine_rows_kernel)
};

// The layer step's projections: Y[M, N] = X[M, K] W[N, K]^T (bf16 in, fp32 accumulation), K a
// multiple of kProjChunk, N a multiple of 64.  K is split into chunks of kProjChunk over workgroups;
// launch_proj_gemm launches the GEMM and the kernel that adds the chunks and applies the epilogue.
constexpr int kProjChunk = 512;
struct ProjArgs {
  const uint16_t* X;      // [M, K] rows of stride x_stride
  int64_t x_stride;
  const uint16_t* W;      // [N, K]
  int32_t M, N, K;
  int32_t norm;           // 1: row m scaled by 1 / sqrt(mean(X[m]^2) + eps) (the input RMSNorm)
  float eps;
  int32_t mode;           // 0: query / kv_a projection; 1: output projection
  // mode 0: outputs n < n_split to y0 [M, n_split] in bf16 (the queries), the rest to y1 [M, N - n_split]
  // in fp32 (the [c_kv | k_pe] rows the cache write reads)
  int32_t n_split;
  uint16_t* y0;
  float* y1;
  // mode 1: out [M, N] in bf16 = Y (+ R, the residual stream, when R is not null)
  const uint16_t* R;
  uint16_t* out;
  // workspace: fp32 partial tiles [m tiles][N / 64][K / kProjChunk][64 x 64] and the chunks' per-token
  // sums of squares [m tiles][K / kProjChunk][64]
  float* part;
  float* ss_part;
};

// ------------------------------------------------------------------------------ launchers

hipError_t launch_absorb(bool bf16, const AbsorbArgs& a, hipStream_t s);
hipError_t launch_cache_write(bool bf16, const CacheWriteArgs& a, hipStream_t s);
hipError_t launch_cache_write_fp8(const CacheWriteArgs& a, hipStream_t s);  // bf16 inputs, fp8 rows
hipError_t launch_q_absorb(bool bf16, const QAbsorbArgs& a, hipStream_t s);
// one launch: the cache write cw (bf16 inputs; bf16 rows, or FP8 rows when fp8) beside the bf16 query
// absorption a
hipError_t launch_decode_prep(const QAbsorbArgs& a, const CacheWriteArgs& cw, bool fp8, hipStream_t s);
// waves: waves per workgroup of the bf16 decode kernel (ignored in fp32 mode)
hipError_t launch_decode(bool bf16, const DecodeArgs& a, int waves, hipStream_t s);
hipError_t launch_decode_f32(const DecodeArgs& a, hipStream_t s);
// FP8 cache rows (kFp8Row bytes), 16-row tiles; every H multiple of 16 and every q_len
hipError_t launch_decode_fp8(const DecodeArgs& a, int waves, hipStream_t s);
// fp8: the cache holds FP8 rows (kFp8Row bytes) instead of bf16 rows; they are first dequantised into a.lat
hipError_t launch_prefill_expand(PrefillArgs a, bool fp8, hipStream_t s);
hipError_t launch_prefill_attn(PrefillArgs a, hipStream_t s);
hipError_t launch_prefill_attn32(PrefillArgs a, hipStream_t s);
hipError_t launch_prefill_qprep(PrefillArgs a, hipStream_t s);
// bf16, 32-row tiles (H*q_len a multiple of 32), T in {1, 2, 4} tiles per workgroup; n_rt = tiles of
// 32 rows per sequence (a multiple of T); units = workgroups, enough that every workgroup's share
// is at most kMt32MaxSteps steps of two blocks
constexpr int kMt32MaxSteps = 1024;
// The 32-row kernel's partition charges each stream this many steps for its setup (query tile,
// pipeline fill, partial store), so that a workgroup that starts several short streams is not
// the last to finish: every workgroup's share, setups included, is at most one setup above the
// mean.
constexpr int kPieceCost = 6;
hipError_t launch_decode_mt32(const DecodeArgs& a, int T, hipStream_t s);
hipError_t launch_combine(bool bf16, const CombineArgs& a, hipStream_t s);
// dst [rows, K] = src [rows, K] * gamma [K] (bf16, rounded once), or a copy when gamma is null
hipError_t launch_layer_pack(const void* src, const void* gamma, void* dst, int64_t rows, int K, hipStream_t s);
hipError_t launch_proj_gemm(const ProjArgs& a, hipStream_t s);
// measurement kernels (ceiling.hip)
constexpr int kMfmaChains = 8;       // independent 16x16x32 MFMA chains per wave in mfma_loop_kernel (32x32x16: half)
constexpr int kMfmaLoopGrid = 1024;  // its workgroups (256 threads): four waves per SIMD
hipError_t launch_mfma_loop(int shape, int iters, uint32_t* sink, int grid, hipStream_t s);
hipError_t launch_stream_read(const void* src, int64_t bytes, uint32_t* sink, int grid, hipStream_t s);
hipError_t launch_gather_dma(const DecodeArgs& a, uint32_t* sink, hipStream_t s);

// ------------------------------------------------------------------------------ device helpers

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef short s16x4_t __attribute__((ext_vector_type(4)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

__device__ __forceinline__ bf16x8_t as_bf16x8(uint4 v) { return __builtin_bit_cast(bf16x8_t, v); }

// 16-byte granule as a native vector.  Register arrays of HIP's uint4 struct are copied with memcpy
// and can be left in private memory; arrays of this type stay in registers.
typedef unsigned u32x4_t __attribute__((ext_vector_type(4)));
typedef unsigned u32x2_t __attribute__((ext_vector_type(2)));

// v_mfma_f32_16x16x32_bf16: D[16x16] += A[16x32] B[32x16].  Lane l holds A row l%16 and B column
// l%16, with 8 consecutive K values per lane (K block l/16); D column l%16, rows 4(l/16)..+3.
__device__ __forceinline__ f32x4_t mfma32(uint4 a, uint4 b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(a), as_bf16x8(b), c, 0, 0, 0);
}
// v_mfma_f32_32x32x16_bf16: A lane l = row l % 32, K values 8 (l / 32) .. + 7; B lane l = column l % 32,
// the same K values; D lane l = column l % 32, rows 8 (R / 4) + 4 (l / 32) + R % 4 in register R
__device__ __forceinline__ f32x16_t mfma32x32(u32x4_t a, u32x4_t b, f32x16_t c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a), __builtin_bit_cast(bf16x8_t, b), c,
                                                 0, 0, 0);
}
__device__ __forceinline__ f32x4_t mfma32v(u32x4_t a, u32x4_t b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a), __builtin_bit_cast(bf16x8_t, b), c,
                                                 0, 0, 0);
}

__device__ __forceinline__ float bf16_to_f32(uint16_t b) { return __uint_as_float(uint32_t(b) << 16); }

// float -> bf16, round to nearest even; NaN stays NaN.
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return uint16_t((u >> 16) | 0x40u);
  return uint16_t((u + 0x7fffu + ((u >> 16) & 1u)) >> 16);
}

// Two floats -> packed bf16 pair (low half = lo) with the hardware converter
// (v_cvt_pk_bf16_f32, round to nearest even in the default rounding mode).
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t cvt_pk_bf16(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2_t{lo, hi}), bf16x2_t));
}

// Power of two 2^-k (k >= 0) that brings x (>= 0) below 2^15, so that x * 2^-k fits fp16 with room to
// spare; 1 for x < 2^15.  Exact scaling: it changes no mantissa bit.
__device__ __forceinline__ float fp16_fit_scale(float x) {
  const int E = int((__float_as_uint(x) >> 23) & 0xffu) - 126;  // x < 2^E for normal x
  const int k = E > 15 ? E - 15 : 0;
  return __uint_as_float(uint32_t(127 - (k > 126 ? 126 : k)) << 23);
}

// Two floats -> packed fp16 pair (low half = lo), round to nearest even.
typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t cvt_pk_f16(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2_t{lo, hi}), f16x2_t));
}
__device__ __forceinline__ f32x2_t f16x2_to_f32(uint32_t v) {
  return __builtin_convertvector(__builtin_bit_cast(f16x2_t, v), f32x2_t);
}

// double -> bf16 with a single rounding (nearest even): round to odd at fp32 precision first
// (truncate, then set the sticky bit if anything was lost), then round to nearest even.
// 24 bits >= 8 + 2, so the two steps give the correctly rounded result.
__device__ __forceinline__ uint16_t f64_to_bf16(double x) {
  float f = __double2float_rz(x);
  if (double(f) != x && !__builtin_isnan(x)) f = __uint_as_float(__float_as_uint(f) | 1u);
  return f32_to_bf16(f);
}

// e4m3 codes -> bf16, exactly (every e4m3 value is a bf16 value), with the hardware converter at scale
// 1; byte k of w -> element k
template <bool HI>
__device__ __forceinline__ uint32_t cvt2(uint32_t w) {
  return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.f, HI));
}
__device__ __forceinline__ u32x4_t codes8(u32x2_t c) {
  return u32x4_t{cvt2<false>(c[0]), cvt2<true>(c[0]), cvt2<false>(c[1]), cvt2<true>(c[1])};
}

// Context length of sequence b as the kernels use it: clamped to [q_len, max_seq_len].
__device__ __forceinline__ int clamp_ctx(int v, int q_len, int max_seq_len) {
  return v < q_len ? q_len : (v > max_seq_len ? max_seq_len : v);
}

// ------------------------------------------------------------------------------ HBM -> LDS transfers

typedef __attribute__((address_space(3))) char lds_char_t;
typedef __attribute__((address_space(3))) s16x4_t lds_s16x4_t;
typedef __attribute__((address_space(3))) const u32x4_t lds_u32x4_t;
typedef __attribute__((address_space(3))) u32x2_t lds_u32x2_t;

// One 16-byte global -> LDS transfer per lane (global_load_lds_dwordx4): lane l's data lands at
// lds + 16 l.  Issued from asm so that the compiler does not track it (it would wait for every
// transfer in flight before the next LDS read); the kernels order it themselves with wait_vmcnt
// (and a barrier when another wave reads the data).  Vector-memory loads complete in issue order,
// so the compiler's own vmcnt waits for older loads stay correct.
__device__ __forceinline__ void dma16(const void* src, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(src), "s"(lds) : "memory", "m0");
}

// The same transfer with the non-temporal hint (nt), for bytes a launch reads once: the decode kernels'
// latent blocks.  A streaming read with the hint ran 9-11 % faster on this device (plain loads and LDS
// transfers alike), the lines not being kept for reuse.
__device__ __forceinline__ void dma16_nt(const void* src, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off nt" ::"v"(src), "s"(lds) : "memory", "m0");
}

// s_waitcnt for vector memory only: vmcnt(n), lgkmcnt and expcnt left at their maxima
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt(((N >> 4) << 14) | (15 << 8) | (7 << 4) | (N & 15));
}

// Workgroup barrier ordering LDS only (the wave's own LDS accesses are complete when it arrives).
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }


// acc += a * b (v_mfma_f32_32x32x16_bf16) on an accumulator tile kept in AGPRs (with the builtin the
// allocator may shuttle it through VGPRs).  The compiler does not see this as an MFMA, so the wait
// states it would add are the callers': the tile is next touched several MFMAs later, its VALU readers
// run after a drain (mfma_drain), and operands written by VALU are followed by s_nop before the first
// of these that reads them.
__device__ __forceinline__ void mfma32x32_acc(f32x16_t& acc, u32x4_t a, u32x4_t b) {
  asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+a"(acc) : "v"(a), "v"(b));
}
// wait states after the last such MFMA before VALU reads its accumulator (> 18 for 16 passes)
__device__ __forceinline__ void mfma_drain() { asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7\n\ts_nop 7" ::: "memory"); }

// Reductions over the lane pairs (l, l ^ 16) and (l, l ^ 32) of a wave with v_permlane16_swap and
// v_permlane32_swap (VALU only; a shuffle is an LDS round trip).  Swapping a value with itself leaves
// lane l holding the pair's two values, so both lanes of a pair compute the same result.
__device__ __forceinline__ f32x2_t lane_pair16(float x) {
  const auto s = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return f32x2_t{__uint_as_float(s[0]), __uint_as_float(s[1])};
}
__device__ __forceinline__ f32x2_t lane_pair32(float x) {
  const auto s = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return f32x2_t{__uint_as_float(s[0]), __uint_as_float(s[1])};
}
__device__ __forceinline__ float xor16_max(float x) { const f32x2_t p = lane_pair16(x); return fmaxf(p[0], p[1]); }
__device__ __forceinline__ float xor32_max(float x) { const f32x2_t p = lane_pair32(x); return fmaxf(p[0], p[1]); }
__device__ __forceinline__ float xor16_add(float x) { const f32x2_t p = lane_pair16(x); return p[0] + p[1]; }
__device__ __forceinline__ float xor32_add(float x) { const f32x2_t p = lane_pair32(x); return p[0] + p[1]; }

// acc *= f for an accumulator vector held in AGPRs, element by element where it is called (a plain
// multiply lets the register allocator keep a VGPR copy of every tile, refreshed each iteration).
// The caller drains in-flight MFMAs that write acc before calling.
template <typename V, int N>
__device__ __forceinline__ void acc_scale(V& acc, float f) {
#pragma unroll
  for (int e = 0; e < N; ++e) {
    float x = acc[e], t;
    asm volatile("v_accvgpr_read_b32 %1, %0\n\tv_mul_f32 %1, %2, %1\n\tv_accvgpr_write_b32 %0, %1"
                 : "+a"(x), "=&v"(t)
                 : "v"(f));
    acc[e] = x;
  }
  asm volatile("" : "+a"(acc));
}
}  // namespace mla
