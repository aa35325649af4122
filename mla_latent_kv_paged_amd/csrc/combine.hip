// S6/S7 -- split-KV combine and the W_uv output projection (mini-infer 17 "MLA Attention：从 KV
// Cache 压缩到矩阵吸收", 版本 3: the value up-projection is applied after attention).
// Split j of row (n, h) left (m_j, l_j, acc_j[512]) with m_j in log2 units; the exact softmax
// result is the log-sum-exp merge
//   o_lat = sum_j 2^(m_j - M) acc_j / sum_j 2^(m_j - M) l_j,   M = max_j m_j,
// and then out[n, h, :] = o_lat . W_uv[h]^T.  Splits are merged in index order: deterministic.
// The fp32 path keeps acc_j; the bf16 kernels store o_j = acc_j / l_j in fp16 (divided by a power
// of two ps_j if its largest entry would not fit), merged with the weights 2^(m_j - M) l_j.  A
// split with m_j = -inf saw no token and weighs nothing.
//
// One workgroup per (head, 16 query rows), or per (head, 64 query rows) when there are enough of those
// to fill the chip (combine_rows_kernel, below); merged o_lat rows are staged in LDS.
// bf16 storage: the projection is a batched MFMA GEMM computed transposed,
//   out^T[v, n] = sum_c W_uv[h][v, c] o_lat^T[c, n]   (K = 512, 16 steps of 16x16x32 bf16),
// with o_lat carried as an unevaluated sum of two bf16 values (hi = bf16(o), lo = bf16(o - hi)),
// i.e. about 16 significant bits, so the product loses nothing visible to the output rounding.
// A workgroup owns 16 rows and either all 128 output channels (four waves, 32 each) or, when the
// (head, 16 rows) grid alone would leave CUs idle, a quarter of them (two waves, 16 each); W_uv
// rows are read straight from global memory, issued before the partials (they depend on nothing).
// fp32 storage: the same merge, then W_uv on the vector ALUs.  Both accumulate in fp32.
#include "mla_internal.h"

namespace mla {

__device__ __forceinline__ float ldw(const uint16_t* p, int64_t i) { return bf16_to_f32(p[i]); }
__device__ __forceinline__ float ldw(const float* p, int64_t i) { return p[i]; }
__device__ __forceinline__ void sto(uint16_t* p, int64_t i, float v) { p[i] = f32_to_bf16(v); }
__device__ __forceinline__ void sto(float* p, int64_t i, float v) { p[i] = v; }

template <typename T>
__global__ __launch_bounds__(256) void combine_kernel(CombineArgs a) {
  const int h = blockIdx.x;
  const int r0 = blockIdx.y * 16;
  const int tid = threadIdx.x;
  __shared__ float olat[16][DC];

  for (int r = 0; r < 16; ++r) {
    const int row = r0 + r;
    if (row >= a.n_q) break;
    const int b = row / a.q_len;
    const int ctx = clamp_ctx(a.seq_lens[b], a.q_len, a.max_seq_len);
    const int nblk = (ctx + BLK - 1) / BLK;
    int ns = (nblk + a.split_blocks - 1) / a.split_blocks;
    if (ns > a.n_split) ns = a.n_split;
    const int64_t base = (int64_t(row) * a.H + h) * a.n_split;
    float M = -INFINITY;
    for (int j = 0; j < ns; ++j) M = fmaxf(M, a.part_ml[base + j].x);
    float den = 0.f, num0 = 0.f, num1 = 0.f;
    for (int j = 0; j < ns; ++j) {
      const float2 ml = a.part_ml[base + j];
      if (ml.x == -INFINITY) continue;
      const float wgt = exp2f(ml.x - M);
      den = fmaf(wgt, ml.y, den);
      const float* acc = a.part_acc + (base + j) * DC;
      num0 = fmaf(wgt, acc[tid], num0);
      num1 = fmaf(wgt, acc[tid + 256], num1);
    }
    olat[r][tid] = num0 / den;
    olat[r][tid + 256] = num1 / den;
  }
  __syncthreads();

  const T* wuv = static_cast<const T*>(a.W_uvT) + int64_t(h) * DC * DV;
  const int v = tid & (DV - 1);
  const int rh = (tid >> 7) * 8;
  float o[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) o[i] = 0.f;
  for (int c = 0; c < DC; ++c) {
    const float w = ldw(wuv, int64_t(c) * DV + v);
#pragma unroll
    for (int i = 0; i < 8; ++i) o[i] = fmaf(olat[rh + i][c], w, o[i]);
  }
  T* out = static_cast<T*>(a.out);
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int row = r0 + rh + i;
    if (row < a.n_q) sto(out, (int64_t(row) * a.H + h) * DV + v, o[i]);
  }
}

// LDS tile of 16 rows x 512 bf16 (64 granules of 16 B per row), granule c of row r stored at
// r*64 + (c ^ swz(r)) so that 16 lanes reading one granule column hit distinct bank groups.
__device__ __forceinline__ int o_swz(int r) { return ((r & 7) << 1) | (r >> 3); }

// Merge the partials of rows row0 .. row0 + 3 (rows >= n_q contribute nothing) of head h: the lane's
// channels 8 lane .. 8 lane + 7 of each row's o_lat, as an unevaluated sum of two bf16 values per
// channel (hi = bf16(o), lo = bf16(o - hi)).
__device__ __forceinline__ void merge_rows4(const CombineArgs& a, int h, int row0, int lane, uint32_t (&hw)[4][4],
                                            uint32_t (&lw)[4][4]) {
  // Row rr's partials are base[rr] + j * stride[rr], j < ns[rr] (by split: consecutive slots; by piece:
  // consecutive pieces of its stream).  They are taken in chunks of 4 up to the largest count
  // among the wave's rows; inside a chunk the loads are unconditional (a row's index is clamped to
  // its last partial and the surplus dropped by selection, never by multiplication).  Chunks are
  // merged with a running max.
  int ns[4], stride[4];
  int64_t base[4];
  if (a.piece_tbl) {
    int2 pt[4];
    int rq[4];
#pragma unroll
    for (int rr = 0; rr < 4; ++rr) {
      const int row = row0 + rr;
      const int rowc = row < a.n_q ? row : a.n_q - 1;
      rq[rr] = (rowc % a.q_len) * a.H + h;  // row within the sequence
      pt[rr] = a.piece_tbl[(rowc / a.q_len) * a.n_grp + rq[rr] / a.rows_per_piece];
      // the same for every lane: kept in scalar registers, and so are the partial addresses below
      pt[rr].x = __builtin_amdgcn_readfirstlane(pt[rr].x);
      pt[rr].y = __builtin_amdgcn_readfirstlane(pt[rr].y);
    }
#pragma unroll
    for (int rr = 0; rr < 4; ++rr) {
      base[rr] = int64_t(pt[rr].x) * a.rows_per_piece + rq[rr] % a.rows_per_piece;
      stride[rr] = a.rows_per_piece;
      ns[rr] = (row0 + rr < a.n_q) ? pt[rr].y : 0;
    }
  } else {
    // every split is read (an empty one carries m = -inf and is skipped by selection), so the
    // loads do not wait for the context length
#pragma unroll
    for (int rr = 0; rr < 4; ++rr) {
      const int row = row0 + rr;
      const int rowc = row < a.n_q ? row : a.n_q - 1;
      base[rr] = (int64_t(rowc) * a.H + h) * a.n_split;
      stride[rr] = 1;
      ns[rr] = row < a.n_q ? a.n_split : 0;
    }
  }
  const int ns_max = __builtin_amdgcn_readfirstlane(max(max(ns[0], ns[1]), max(ns[2], ns[3])));
  // a chunk's 16 (m, l) pairs and scales: lane l loads those of row (l / 4) % 4, partial j0 + l % 4, and
  // they reach every lane by readlane (scalar registers instead of 48 vector registers per chunk)
  const int lr = (lane >> 2) & 3, lj = lane & 3;
  const int64_t lbase = lr == 0 ? base[0] : lr == 1 ? base[1] : lr == 2 ? base[2] : base[3];
  const int lstride = lr == 0 ? stride[0] : lr == 1 ? stride[1] : lr == 2 ? stride[2] : stride[3];
  const int lns = lr == 0 ? ns[0] : lr == 1 ? ns[1] : lr == 2 ? ns[2] : ns[3];
  float M[4], den[4], o[4][8];
#pragma unroll
  for (int rr = 0; rr < 4; ++rr) {
    M[rr] = -INFINITY;
    den[rr] = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) o[rr][e] = 0.f;
  }
  for (int j0 = 0; j0 < ns_max; j0 += 4) {
    float2 ml[4][4];
    float ps[4][4];
    u32x4_t vo[4][4];  // fp16 o / ps of channels 8 lane .. 8 lane + 7
    const int64_t lpi = lbase + int64_t(min(j0 + lj, max(lns - 1, 0))) * lstride;
    const float2 lml = a.part_ml[lpi];
    const float lps = a.part_scale[lpi];
#pragma unroll
    for (int rr = 0; rr < 4; ++rr)
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        const int jc = min(j0 + jj, max(ns[rr] - 1, 0));
        const int64_t pi = base[rr] + int64_t(jc) * stride[rr];
        vo[rr][jj] = *reinterpret_cast<const u32x4_t*>(a.part_o16 + pi * DC + 8 * lane);
      }
#pragma unroll
    for (int rr = 0; rr < 4; ++rr)
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        ml[rr][jj].x = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(lml.x), 4 * rr + jj));
        ml[rr][jj].y = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(lml.y), 4 * rr + jj));
        ps[rr][jj] = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(lps), 4 * rr + jj));
      }
#pragma unroll
    for (int rr = 0; rr < 4; ++rr) {
      bool ok[4];
      float mc = M[rr];
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        ok[jj] = j0 + jj < ns[rr] && ml[rr][jj].x != -INFINITY;
        mc = ok[jj] ? fmaxf(mc, ml[rr][jj].x) : mc;
      }
      const float sc = (M[rr] == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(M[rr] - mc);
      den[rr] *= sc;
#pragma unroll
      for (int e = 0; e < 8; ++e) o[rr][e] *= sc;
      M[rr] = mc;
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        if (!ok[jj]) continue;
        // weight of split j: 2^(m_j - M) l_j (its o is already divided by l_j)
        const float wgt = __builtin_amdgcn_exp2f(ml[rr][jj].x - mc) * ml[rr][jj].y;
        den[rr] += wgt;
        const float wo = wgt * ps[rr][jj];  // the stored row is o / ps (a power of two)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const f32x2_t x = f16x2_to_f32(vo[rr][jj][e]);
          o[rr][2 * e] = fmaf(wo, x[0], o[rr][2 * e]);
          o[rr][2 * e + 1] = fmaf(wo, x[1], o[rr][2 * e + 1]);
        }
      }
    }
  }
#pragma unroll
  for (int rr = 0; rr < 4; ++rr) {
    const float inv = den[rr] > 0.f ? 1.f / den[rr] : 0.f;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float x0 = o[rr][2 * e] * inv, x1 = o[rr][2 * e + 1] * inv;
      hw[rr][e] = cvt_pk_bf16(x0, x1);
      lw[rr][e] = cvt_pk_bf16(x0 - __uint_as_float(hw[rr][e] << 16), x1 - __uint_as_float(hw[rr][e] & 0xffff0000u));
    }
  }
}

__global__ __launch_bounds__(256) void combine_bf16_kernel(CombineArgs a) {
  const int h = blockIdx.x;
  const int r0 = blockIdx.y * 16;
  const int vq = blockIdx.z;  // part of the 128 output channels (one of v_parts)
  const int tid = threadIdx.x;
  const int lane = tid & 63, w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform
  __shared__ uint4 ohi[16 * 64];
  __shared__ uint4 olo[16 * 64];

  // output channel tiles of 16: with 4 parts, waves 0 and 1 take one tile each of this
  // workgroup's 32 channels; with 1 part, every wave takes two tiles of its 32.  The first tile's
  // W_uv fragments do not depend on the merge, so their loads are issued first.
  const int ntile = a.v_parts == 1 ? 2 : 1;
  const int vbase = a.v_parts == 1 ? 32 * w : vq * 32 + (w & 1) * 16;
  const uint16_t* wuv_h = static_cast<const uint16_t*>(a.W_uv) + int64_t(h) * DV * DC;
  const uint4* wrow = reinterpret_cast<const uint4*>(wuv_h + int64_t(vbase + (lane & 15)) * DC);
  const bool gemm_wave = a.v_parts == 1 || w < 2;
  uint4 wf[16];
  if (gemm_wave) {
#pragma unroll
    for (int ks = 0; ks < 16; ++ks) wf[ks] = wrow[4 * ks + (lane >> 4)];
  }

  // merge the partials: wave w owns rows 4w..4w+3
  {
    uint32_t hw[4][4], lw[4][4];
    merge_rows4(a, h, r0 + w * 4, lane, hw, lw);
#pragma unroll
    for (int rr = 0; rr < 4; ++rr) {
      const int r = w * 4 + rr;
      const int gi = r * 64 + (lane ^ o_swz(r));
      ohi[gi] = make_uint4(hw[rr][0], hw[rr][1], hw[rr][2], hw[rr][3]);
      olo[gi] = make_uint4(lw[rr][0], lw[rr][1], lw[rr][2], lw[rr][3]);
    }
  }
  __syncthreads();
  if (a.v_parts != 1 && w >= 2) return;

  // out^T[v, n] for 16 output channels v per tile and the 16 rows n of this workgroup
  const int r16 = lane & 15, g = lane >> 4;
  const int row = r0 + r16;
  for (int t = 0; t < ntile; ++t) {
    if (t > 0) {
      const uint4* wr = reinterpret_cast<const uint4*>(wuv_h + int64_t(vbase + 16 * t + (lane & 15)) * DC);
#pragma unroll
      for (int ks = 0; ks < 16; ++ks) wf[ks] = wr[4 * ks + (lane >> 4)];
    }
    f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < 16; ++ks) {
      const int c = 4 * ks + g;
      acc = mfma32(wf[ks], ohi[r16 * 64 + (c ^ o_swz(r16))], acc);
      acc = mfma32(wf[ks], olo[r16 * 64 + (c ^ o_swz(r16))], acc);
    }
    // lane holds query row r0 + r16 (column), output channels vbase + 16t + 4g .. +3 (rows)
    if (row < a.n_q) {
      uint16_t* out = static_cast<uint16_t*>(a.out) + (int64_t(row) * a.H + h) * DV + vbase + 16 * t + 4 * g;
      *reinterpret_cast<uint2*>(out) = make_uint2(cvt_pk_bf16(acc[0], acc[1]), cvt_pk_bf16(acc[2], acc[3]));
    }
  }
}

// Many rows per head (the wide and multi-token shapes): one workgroup per (head, RW query rows) with RW / 4
// waves, so that W_uv[h] is read once per RW rows instead of once per 16.  Wave w merges rows 4w .. 4w + 3 as
// above.  The product out^T[v, n] = sum_c W_uv[h][v, c] o_lat^T[c, n] then runs on v_mfma_f32_32x32x16_bf16
// with the 512 channels c cut into KQ = RW / 16 parts: wave w takes output channels 32 (w % 4) .. + 31 over
// channel part w / 4, for every 32-row column tile, on the hi and on the lo half of o_lat.  The parts' fp32
// sums meet in LDS, are added in part order and stored as bf16, 16 bytes per lane.
template <int RW>
__global__ __launch_bounds__(RW * 16) void combine_rows_kernel(CombineArgs a) {
  constexpr int KQ = RW / 16, NT = RW / 32, NKS = 32 / KQ;  // channel parts, column tiles, K steps per wave
  constexpr int kRed = DV + 4;  // floats per row of the parts' sums (rows start 16 bytes apart in bank terms)
  constexpr int kLdsO = 2 * RW * 64 * 16;  // the hi and lo tiles: RW rows of 64 granules of 16 bytes each
  constexpr int kLdsR = KQ * RW * kRed * 4;
  __shared__ __attribute__((aligned(16))) char lds[kLdsO > kLdsR ? kLdsO : kLdsR];
  u32x4_t* ohi = reinterpret_cast<u32x4_t*>(lds);  // granule c of row r at r * 64 + (c ^ (r % 16))
  u32x4_t* olo = ohi + RW * 64;
  float* red = reinterpret_cast<float*>(lds);  // [KQ][RW][kRed], after the product

  const int h = blockIdx.x, r0 = blockIdx.y * RW;
  const int tid = threadIdx.x, lane = tid & 63, w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int vt = w & 3, kq = w >> 2, hf = lane >> 5;

  const uint16_t* wuv_h = static_cast<const uint16_t*>(a.W_uv) + int64_t(h) * DV * DC;
  const u32x4_t* wrow = reinterpret_cast<const u32x4_t*>(wuv_h + int64_t(32 * vt + (lane & 31)) * DC) + 2 * NKS * kq;
  u32x4_t wf[NKS];
  {
    uint32_t hw[4][4], lw[4][4];
    merge_rows4(a, h, r0 + 4 * w, lane, hw, lw);
    // the W_uv fragments, issued once the merge's registers are free (their latency overlaps the
    // barrier): the A operand of K step ks is row 32 vt + lane % 32, channels 16 (kq NKS + ks) + 8 hf .. + 7
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) wf[ks] = wrow[2 * ks + hf];
#pragma unroll
    for (int rr = 0; rr < 4; ++rr) {
      const int r = 4 * w + rr;
      const int gi = r * 64 + (lane ^ (r & 15));
      ohi[gi] = u32x4_t{hw[rr][0], hw[rr][1], hw[rr][2], hw[rr][3]};
      olo[gi] = u32x4_t{lw[rr][0], lw[rr][1], lw[rr][2], lw[rr][3]};
    }
  }
  __syncthreads();

  f32x16_t acc[NT];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) acc[nt] = f32x16_t{};
#pragma unroll
  for (int ks = 0; ks < NKS; ++ks) {
    const int g = 2 * (NKS * kq + ks) + hf;  // the B operand's granule: the same channels as wf[ks]
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      const int n = 32 * nt + (lane & 31);
      const int gi = n * 64 + (g ^ (n & 15));
      acc[nt] = mfma32x32(wf[ks], ohi[gi], acc[nt]);
      acc[nt] = mfma32x32(wf[ks], olo[gi], acc[nt]);
    }
  }
  __syncthreads();  // the tiles' memory takes the parts' sums

  // lane holds column n = 32 nt + lane % 32 (a query row) and, in register 4q + i, output channel
  // 32 vt + 8q + 4 hf + i
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    float* dst = red + (kq * RW + 32 * nt + (lane & 31)) * kRed + 32 * vt + 4 * hf;
#pragma unroll
    for (int q = 0; q < 4; ++q)
      *reinterpret_cast<f32x4_t*>(dst + 8 * q) = f32x4_t{acc[nt][4 * q], acc[nt][4 * q + 1], acc[nt][4 * q + 2],
                                                          acc[nt][4 * q + 3]};
  }
  __syncthreads();

  // thread: row n = tid / 16, output channels 8 (tid % 16) .. + 7
  const int n = tid >> 4, v0 = 8 * (tid & 15);
  f32x4_t s0 = {0.f, 0.f, 0.f, 0.f}, s1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int p = 0; p < KQ; ++p) {
    const float* src = red + (p * RW + n) * kRed + v0;
    s0 += *reinterpret_cast<const f32x4_t*>(src);
    s1 += *reinterpret_cast<const f32x4_t*>(src + 4);
  }
  const int row = r0 + n;
  if (row < a.n_q) {
    uint16_t* out = static_cast<uint16_t*>(a.out) + (int64_t(row) * a.H + h) * DV + v0;
    *reinterpret_cast<u32x4_t*>(out) = u32x4_t{cvt_pk_bf16(s0[0], s0[1]), cvt_pk_bf16(s0[2], s0[3]),
                                                 cvt_pk_bf16(s1[0], s1[1]), cvt_pk_bf16(s1[2], s1[3])};
  }
}

hipError_t launch_combine(bool bf16, const CombineArgs& a, hipStream_t s) {
  if (bf16 && a.rows_wg == 64) {
    launch(combine_rows_kernel<64>, dim3(a.H, (a.n_q + 63) / 64), dim3(64 * 16), 0, s, a);
  } else if (bf16) {
    dim3 grid(a.H, (a.n_q + 15) / 16, a.v_parts);
    launch(combine_bf16_kernel, dim3(grid), dim3(256), 0, s, a);
  } else {
    dim3 grid(a.H, (a.n_q + 15) / 16);
    launch(combine_kernel<float>, dim3(grid), dim3(256), 0, s, a);
  }
  return hipGetLastError();
}

}  // namespace mla
