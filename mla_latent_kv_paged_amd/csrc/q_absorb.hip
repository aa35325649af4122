// S2 -- query side of the absorbed decode (mini-infer 17 "MLA Attention：从 KV Cache 压缩到矩阵吸收",
// 版本 3 and 设计取舍; vLLM learning book ch. 07 §2.4 Decoupled RoPE):
//   q_lat[n,h,:] = q_nope[n,h,:] . W_uk[h]            (W_uk folded into the query, DC values)
//   q_pe'[n,h,:] = RoPE(q_pe[n,h,:], p_n),  p_n = ctx_b - q_len + i  for row n = b*q_len + i
// Both are scaled by softmax_scale*log2(e) so that the decode kernel works in log2 units, and
// stored as one [q_lat | q_pe'] row of 576 values per (n, h) in the storage dtype.
//
// bf16 storage: a batched MFMA GEMM per head, computed transposed so that each lane stores four
// consecutive channels: q_lat^T[c, n] = sum_k W_uk^T[c, k] q_nope^T[k, n], K = 128 (4 steps of
// v_mfma_f32_16x16x32_bf16).  A workgroup owns 64 query rows of one head (each wave 16 rows, their
// q_nope loaded once) and half of the 512 channels, or less when the grid would otherwise be too
// small to fill the chip; its W_uk^T slice is staged in LDS with one batch of loads.
// fp32 storage: one workgroup per (head, 16 query rows) on the vector ALUs, W_uk[h] streamed once
// per workgroup, each thread owning two latent columns.  Both accumulate in fp32.
// The decode step's first launch (decode_prep_kernel) adds the new tokens' cache-write workgroups
// to the bf16 grid: the two steps are independent and latency-bound at decode sizes.
#include "cache_write_impl.h"

namespace mla {

__device__ __forceinline__ float ld(const uint16_t* p, int64_t i) { return bf16_to_f32(p[i]); }
__device__ __forceinline__ float ld(const float* p, int64_t i) { return p[i]; }
__device__ __forceinline__ void st(uint16_t* p, int64_t i, float v) { p[i] = f32_to_bf16(v); }
__device__ __forceinline__ void st(float* p, int64_t i, float v) { p[i] = v; }

// RoPE of q_pe for one (row, head, pair), fp64 then scaled and rounded once.
__device__ __forceinline__ void rope_q_pair(const QAbsorbArgs& a, int row, int h, int i, float x0f, float x1f,
                                            float* y0, float* y1) {
  const int b = row / a.q_len, iq = row % a.q_len;
  const int ctx = clamp_ctx(a.seq_lens[b], a.q_len, a.max_seq_len);
  const int pos = ctx - a.q_len + iq;
  *y0 = __builtin_nanf("");
  *y1 = __builtin_nanf("");
  if (pos >= 0 && pos <= a.max_position) {
    const double2 cs = a.rope[int64_t(pos) * NPAIR + i];
    const double x0 = x0f, x1 = x1f;
    *y0 = float((x0 * cs.x - x1 * cs.y) * double(a.qscale));
    *y1 = float((x0 * cs.y + x1 * cs.x) * double(a.qscale));
  }
}

template <typename T>
__global__ __launch_bounds__(256) void q_absorb_kernel(QAbsorbArgs a) {
  const int h = blockIdx.x;
  const int r0 = blockIdx.y * 16;
  const int tid = threadIdx.x;
  const T* q = static_cast<const T*>(a.q);
  const T* wuk = static_cast<const T*>(a.W_uk) + int64_t(h) * DN * DC;
  T* qcat = static_cast<T*>(a.qcat);

  __shared__ float qn[16][DN];
  __shared__ float qp[16][DR];
  for (int idx = tid; idx < 16 * QW; idx += 256) {
    const int r = idx / QW, d = idx % QW;
    const int row = r0 + r;
    const float v = row < a.n_q ? ld(q, (int64_t(row) * a.H + h) * QW + d) : 0.f;
    if (d < DN)
      qn[r][d] = v;
    else
      qp[r][d - DN] = v;
  }
  __syncthreads();

  float acc0[16], acc1[16];
#pragma unroll
  for (int r = 0; r < 16; ++r) acc0[r] = acc1[r] = 0.f;
  for (int n = 0; n < DN; ++n) {
    const float w0 = ld(wuk, int64_t(n) * DC + tid);
    const float w1 = ld(wuk, int64_t(n) * DC + tid + 256);
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      acc0[r] = fmaf(qn[r][n], w0, acc0[r]);
      acc1[r] = fmaf(qn[r][n], w1, acc1[r]);
    }
  }
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const int row = r0 + r;
    if (row < a.n_q) {
      T* o = qcat + (int64_t(row) * a.H + h) * ROW;
      st(o, tid, acc0[r] * a.qscale);
      st(o, tid + 256, acc1[r] * a.qscale);
    }
  }

  // RoPE on q_pe at the query position, evaluated in fp64 then scaled and rounded once.
  for (int idx = tid; idx < 16 * NPAIR; idx += 256) {
    const int r = idx / NPAIR, i = idx % NPAIR;
    const int row = r0 + r;
    if (row >= a.n_q) continue;
    float y0, y1;
    rope_q_pair(a, row, h, i, qp[r][2 * i], qp[r][2 * i + 1], &y0, &y1);
    T* o = qcat + (int64_t(row) * a.H + h) * ROW + DC;
    st(o, 2 * i, y0);
    st(o, 2 * i + 1, y1);
  }
}

// workgroup (head h, 64 query rows rb, channel part cp of c_split); wlds: 64 KiB of LDS
__device__ __forceinline__ void q_absorb_bf16_block(const QAbsorbArgs& a, int c_split, int h, int rb, int cp,
                                                    u32x4_t* wlds) {
  const int lane = threadIdx.x & 63, w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int r16 = lane & 15, g = lane >> 4;
  const uint16_t* q = static_cast<const uint16_t*>(a.q);
  uint16_t* qcat = static_cast<uint16_t*>(a.qcat);
  // B operand: q_nope of this wave's 16 rows (granule 4 ks + g of the 128-wide row), loaded once;
  // rows past n_q read row 0 and are not stored
  const int n = rb * 64 + 16 * w + r16;
  const bool nv = n < a.n_q;
  const u32x4_t* qrow = reinterpret_cast<const u32x4_t*>(q + (int64_t(nv ? n : 0) * a.H + h) * QW);
  u32x4_t bq[4];
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) bq[ks] = qrow[4 * ks + g];
  // RoPE inputs, loaded before the GEMM so that their two dependent round trips overlap it: the
  // c_split workgroups of this (head, 64 rows) share the rows, each thread taking ppt consecutive
  // pairs of one row (one context-length load, then contiguous q_pe values and table entries)
  const int ppt = 8 / c_split;  // pairs per thread (4, 2 or 1)
  const int tpr = NPAIR / ppt;  // threads per row
  const int nr = rb * 64 + cp * (64 / c_split) + int(threadIdx.x) / tpr;
  const int i0 = (int(threadIdx.x) % tpr) * ppt;
  const bool rv = nr < a.n_q;
  uint32_t rq[4] = {0u, 0u, 0u, 0u};
  double2 rc[4] = {};
  bool rok = false;
  uint16_t* ro = qcat + (int64_t(rv ? nr : 0) * a.H + h) * ROW + DC + 2 * i0;
  if (rv) {
    const int ctx = clamp_ctx(a.seq_lens[nr / a.q_len], a.q_len, a.max_seq_len);
    const int pos = ctx - a.q_len + nr % a.q_len;
    rok = pos >= 0 && pos <= a.max_position;
    const uint32_t* src = reinterpret_cast<const uint32_t*>(q + (int64_t(nr) * a.H + h) * QW + DN + 2 * i0);
    const double2* cs = a.rope + int64_t(rok ? pos : 0) * NPAIR + i0;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      if (e < ppt) {
        rq[e] = src[e];
        rc[e] = cs[e];
      }
    }
  }
  // A operand: this workgroup's W_uk^T rows (NC channels x 16 granules).  64 channels go straight
  // into registers; more are staged in LDS with one batch of loads, granule gi of row r at
  // r*16 + (gi ^ (r % 16)), so that the 16 rows of a tile read at one granule column hit distinct
  // bank groups
  const int NC = DC / c_split;  // <= 256
  const int ntile = NC / 16;
  const int c_first = cp * NC;
  uint16_t* orow = qcat + (int64_t(nv ? n : 0) * a.H + h) * ROW + c_first + 4 * g;
  if (c_split == 8) {
    // 64 channels: each wave's four tiles straight from global memory, all loads in flight together
    // (a small grid is latency-bound; staging through LDS would add a round trip)
    const u32x4_t* wt = reinterpret_cast<const u32x4_t*>(static_cast<const uint16_t*>(a.W_ukT) +
                                                       (int64_t(h) * DC + c_first + r16) * DN);
    u32x4_t af[4][4];
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) af[t][ks] = wt[t * 16 * (DN / 8) + 4 * ks + g];
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) acc = mfma32v(af[t][ks], bq[ks], acc);
      if (nv)
        *reinterpret_cast<uint2*>(orow + 16 * t) =
            make_uint2(cvt_pk_bf16(acc[0] * a.qscale, acc[1] * a.qscale), cvt_pk_bf16(acc[2] * a.qscale, acc[3] * a.qscale));
    }
  } else {
    {
      const u32x4_t* wsrc = reinterpret_cast<const u32x4_t*>(static_cast<const uint16_t*>(a.W_ukT) +
                                                           (int64_t(h) * DC + c_first) * DN);
      const int cnt = NC * 16 / 256;  // granules per thread (16 or 8)
      u32x4_t tmp[16];  // native vectors: plain loads and stores, the array stays in registers
#pragma unroll
      for (int k = 0; k < 16; ++k)
        if (k < cnt) tmp[k] = wsrc[threadIdx.x + 256 * k];
#pragma unroll
      for (int k = 0; k < 16; ++k)
        if (k < cnt) {
          const int e = threadIdx.x + 256 * k, r = e >> 4, gi = e & 15;
          wlds[r * 16 + (gi ^ (r & 15))] = tmp[k];
        }
    }
    __syncthreads();
    // all tiles first (lane: query row n, channels c_first + 16 t + 4g .. + 3), packed to bf16
    uint2 pk[16];
#pragma unroll
    for (int t = 0; t < 16; ++t) {
      if (t < ntile) {
        const int r = 16 * t + r16;
        f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) acc = mfma32v(wlds[r * 16 + ((4 * ks + g) ^ r16)], bq[ks], acc);
        pk[t] = make_uint2(cvt_pk_bf16(acc[0] * a.qscale, acc[1] * a.qscale), cvt_pk_bf16(acc[2] * a.qscale, acc[3] * a.qscale));
      }
    }
    // then through LDS (every wave is done with W_uk^T), so that the rows are stored 16 contiguous bytes
    // per lane: whole cache lines, not 8-byte pieces of 16 rows.  Wave w's rows at w * 16 * NC channels,
    // granule gi of row r16 at gi ^ r16 (the 16 lanes of a granule column hit distinct bank groups)
    __syncthreads();
    uint2* ot = reinterpret_cast<uint2*>(wlds) + w * 16 * (NC / 4);  // 4 channels per uint2
    const int gpr = NC / 8;                                          // 16-byte granules per row (32 or 16)
#pragma unroll
    for (int t = 0; t < 16; ++t) {
      if (t < ntile) {
        const int gi = 2 * t + (g >> 1);  // channels 16 t + 4 g: granule 2 t + g / 2, half g % 2
        ot[r16 * (NC / 4) + 2 * (gi ^ (r16 & (gpr - 1))) + (g & 1)] = pk[t];
      }
    }
    __builtin_amdgcn_s_waitcnt(0xc07f);  // this wave's LDS writes are done (lgkmcnt(0)); it reads only its own rows
    const u32x4_t* orl = reinterpret_cast<const u32x4_t*>(ot);
    for (int e = lane; e < 16 * gpr; e += 64) {
      const int rr = e / gpr, gi = e % gpr;
      const int nn = rb * 64 + 16 * w + rr;
      if (nn < a.n_q)
        *reinterpret_cast<u32x4_t*>(qcat + (int64_t(nn) * a.H + h) * ROW + c_first + 8 * gi) =
            orl[rr * gpr + (gi ^ (rr & (gpr - 1)))];
    }
  }
  // RoPE part: results computed and stored after the GEMM from the values loaded above, the thread's
  // ppt pairs in one store (its 4 ppt contiguous bytes)
  if (rv) {
    u32x4_t y = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      if (e < ppt) {
        const double x0 = bf16_to_f32(rq[e] & 0xffffu), x1 = bf16_to_f32(rq[e] >> 16);
        const float y0 = rok ? float((x0 * rc[e].x - x1 * rc[e].y) * double(a.qscale)) : __builtin_nanf("");
        const float y1 = rok ? float((x0 * rc[e].y + x1 * rc[e].x) * double(a.qscale)) : __builtin_nanf("");
        y[e] = cvt_pk_bf16(y0, y1);
      }
    }
    if (ppt == 4)
      *reinterpret_cast<u32x4_t*>(ro) = y;
    else if (ppt == 2)
      *reinterpret_cast<u32x2_t*>(ro) = u32x2_t{y[0], y[1]};
    else
      *reinterpret_cast<uint32_t*>(ro) = y[0];
  }
}

__global__ __launch_bounds__(256) void q_absorb_bf16_kernel(QAbsorbArgs a, int c_split) {
  __shared__ u32x4_t wlds[256 * 16];  // up to 256 channels of W_uk^T (64 KiB)
  q_absorb_bf16_block(a, c_split, blockIdx.x, blockIdx.y, blockIdx.z, wlds);
}

// The decode step's first launch: the two independent steps before the decode kernel in one grid.
// Workgroups 0 .. ncw - 1 write the new tokens' cache rows (four tokens each, FP8 rows when fp8; from
// fp32 inputs for the layer step); the rest are the query absorption's (head, 64 rows, channel part),
// in its own order.
__global__ __launch_bounds__(256) void decode_prep_kernel(QAbsorbArgs a, int c_split, CacheWriteArgs cw, int ncw,
                                                          int fp8) {
  __shared__ u32x4_t wlds[256 * 16];
  const int bid = int(blockIdx.x);
  if (bid < ncw) {
    const int j = bid * 4 + int(threadIdx.x >> 6);
    if (fp8) {
      if (cw.in_f32)
        cache_write_fp8_token<float>(cw, j, threadIdx.x & 63);
      else
        cache_write_fp8_token<uint16_t>(cw, j, threadIdx.x & 63);
    } else {
      if (cw.in_f32)
        cache_write_token<uint16_t, float>(cw, j, threadIdx.x & 63);
      else
        cache_write_token<uint16_t>(cw, j, threadIdx.x & 63);
    }
    return;
  }
  const int q = bid - ncw;
  const int rbs = (a.n_q + 63) / 64;
  q_absorb_bf16_block(a, c_split, q % a.H, (q / a.H) % rbs, q / (a.H * rbs), wlds);
}

namespace {
// channels split over c_split workgroups only as far as needed for about 512 workgroups; at most
// 256 channels per workgroup (its W_uk^T slice fits 64 KiB of LDS)
int q_absorb_c_split(const QAbsorbArgs& a) {
  const int rbs = (a.n_q + 63) / 64;
  int c_split = 2;
  while (c_split < 8 && int64_t(a.H) * rbs * c_split < 512) c_split *= 2;
  return c_split;
}
}  // namespace

hipError_t launch_decode_prep(const QAbsorbArgs& a, const CacheWriteArgs& cw, bool fp8, hipStream_t s) {
  const int c_split = q_absorb_c_split(a);
  const int64_t ncw = cw.T > 0 ? (int64_t(cw.T) + 3) / 4 : 0;
  const int64_t grid = ncw + int64_t(a.H) * ((a.n_q + 63) / 64) * c_split;
  if (grid > 0x7fffffff) return hipErrorInvalidValue;
  launch(decode_prep_kernel, dim3(int(grid)), dim3(256), 0, s, a, c_split, cw, int(ncw), fp8 ? 1 : 0);
  return hipGetLastError();
}

hipError_t launch_q_absorb(bool bf16, const QAbsorbArgs& a, hipStream_t s) {
  if (bf16) {
    const int c_split = q_absorb_c_split(a);
    dim3 grid(a.H, (a.n_q + 63) / 64, c_split);
    launch(q_absorb_bf16_kernel, dim3(grid), dim3(256), 0, s, a, c_split);
  } else {
    dim3 grid(a.H, (a.n_q + 15) / 16);
    launch(q_absorb_kernel<float>, dim3(grid), dim3(256), 0, s, a);
  }
  return hipGetLastError();
}

}  // namespace mla
