// S3-S6 over an FP8 latent cache -- split-KV paged MLA decode, 16 query rows per sequence and split.
//
// What is computed: the same as decode_bf16.hip (mini-infer 17 "MLA Attention：从 KV Cache 压缩到矩阵吸收",
// 版本 3 and 设计取舍; 踩坑记录 坑 2 causal mask; vLLM learning book ch. 07 §2.3 paged cache shape;
// bxzpzcl.cn hybrid KV-cache page §2.1 block table), over cache rows that hold the normed latent
// as FP8 E4M3 codes in 4 groups of 128 channels with one fp32 scale per group (the vLLM learning
// book, ch. 07, lists an FP8 KV cache for MLA; the row layout and scale rule are this library's):
//   row (656 B) = [ 512 codes | 64 bf16 rope values | 4 fp32 scales ],  c_i = e4m3(code_i) * s_{i/128}
// Nothing is rounded on the way in: codes convert to bf16 exactly (e4m3 is a subset of bf16) and
// the scales are applied in fp32 to the MFMA results:
//   s[r,t] = sum_g s_{t,g} (q_lat[r, g] . code_t[g]) + q_pe'[r] . k_pe_t          (scores)
//   acc[r, g] += sum_t (P[r,t] s_{t,g}) code_t[g]                                  (P.C)
// with P[r,t] s_{t,g} rounded to bf16 as the MFMA operand, as P alone is in the bf16 kernel.
//
// How:
//  * A paged block is 16 rows of 656 bytes = 10,496 contiguous bytes.  Each wave streams its blocks
//    HBM -> LDS with global_load_lds_dwordx4 (11 transfers of 1 KB, the last one partly into padding)
//    into a private ring of NS stages, NS - 1 blocks ahead.
//  * Per block, the wave converts its stage into a bf16 tile in the layout of the bf16 kernel (8 x 8
//    chunks of 16-byte granules): v_cvt_scalef32_pk_bf16_fp8 with scale 1 for the codes (exact),
//    a copy for the rope granules, zeros for tokens past the visible range.  From there the scores
//    (v_mfma_f32_16x16x32_bf16, A by ds_read_b128) and P.C (v_mfma_f32_16x16x16_bf16, A by
//    ds_read_b64_tr_b16) run as in the bf16 kernel, with the group scales of the lane's four
//    tokens read once per block.
//  * Merge, normalisation and the fp16 partial store are those of the bf16 kernel.
#include "mla_internal.h"

namespace mla {

namespace {

constexpr int kTileBytes = BLK * ROW * 2;        // a bf16 tile of 16 rows x 576 (block or query tile)
constexpr int kStage8 = 11 * 1024;               // fp8 stage: one block (10,496 B) + transfer padding
constexpr float kMaxSlack = 8.f;                 // lazy-rescale slack, as in the bf16 kernel

__device__ __forceinline__ void wait_blocks8(int n) {  // at most n blocks (11 transfers each) in flight
  if (n <= 0)
    wait_vmcnt<0>();
  else if (n == 1)
    wait_vmcnt<11>();
  else if (n == 2)
    wait_vmcnt<22>();
  else
    wait_vmcnt<33>();
}

}  // namespace

template <int NW, int NS>
__global__ __launch_bounds__(NW * 64) void decode_fp8_kernel(DecodeArgs a) {
  static_assert(NW == 2, "the query tile is moved by two waves");
  static_assert(NS >= 2 && NS <= 4, "a wave keeps at most 3 blocks in flight");
  static_assert(NW * NS * kStage8 >= 32 * 64 * 16 + 16 * 1024, "the merge reuses the rings");
  __shared__ __attribute__((aligned(16))) char ring_mem[NW * NS * kStage8];
  __shared__ __attribute__((aligned(16))) char tile_mem[NW * kTileBytes];
  __shared__ __attribute__((aligned(16))) char q_mem[kTileBytes];
  __shared__ float m_lds[NW][16];
  __shared__ float l_lds[NW][16];
  __shared__ float x_lds[NW][16];

  // work unit u = (sequence b, split j, row tile rt), rt fastest; contiguous unit ranges per XCD
  const int per_xcd = (a.units + 7) >> 3;
  const int u = int(blockIdx.x & 7) * per_xcd + int(blockIdx.x >> 3);
  if (u >= a.units) return;
  const int rt = u % a.n_rt;
  const int j = (u / a.n_rt) % a.n_split;
  const int b = u / (a.n_rt * a.n_split);

  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int r16 = lane & 15;
  const int g = lane >> 4;
  const int lrow = lane & 7, lgr = lane >> 3;

  const int tiles_per_q = a.H >> 4;
  const int iq = rt / tiles_per_q;
  const int h0 = (rt % tiles_per_q) << 4;
  const int row = b * a.q_len + iq;
  const int kb0 = j * a.split_blocks;
  const char* cache = static_cast<const char*>(a.cache);
  const char* zero = static_cast<const char*>(a.zero_block);  // >= 10,496 zero bytes
  lds_char_t* const ring = (lds_char_t*)ring_mem + w * (NS * kStage8);
  lds_char_t* const tile = (lds_char_t*)tile_mem + w * kTileBytes;

  // start-up as in the bf16 kernel: context length, block ids and query tile requested together
  const int ctx = clamp_ctx(a.seq_lens[b], a.q_len, a.max_seq_len);
  const int* bt = a.block_table + int64_t(b) * a.bt_stride;
  const int in_row = min(a.split_blocks, a.bt_stride - kb0) - w;
  const int nid = in_row > 0 ? (in_row + NW - 1) / NW : 0;
  const int phys_lo = lane < nid ? bt[kb0 + w + NW * lane] : 0;
  const int phys_hi = lane + 64 < nid ? bt[kb0 + w + NW * (lane + 64)] : 0;
  {  // query tile -> LDS: wave w moves rows 8w..8w+7
    const char* src = static_cast<const char*>(a.qcat) + (int64_t(row) * a.H + h0 + 8 * w + lrow) * (ROW * 2) +
                      16 * lgr;
    const uint32_t dst = __builtin_amdgcn_readfirstlane(uint32_t(uintptr_t((lds_char_t*)q_mem)));
#pragma unroll
    for (int gq = 0; gq < 9; ++gq) dma16(src + 128 * gq, dst + 1024 * (9 * w + gq));
  }
  asm volatile("" ::"v"(phys_lo), "v"(phys_hi));  // the ids are complete (see decode_bf16.hip)
  auto phys_of = [&](int i) {
    return i < 64 ? __builtin_amdgcn_readlane(phys_lo, i & 63) : __builtin_amdgcn_readlane(phys_hi, i & 63);
  };

  const int nblk = (ctx + BLK - 1) / BLK;
  const int ns = (nblk + a.split_blocks - 1) / a.split_blocks;
  if (j >= ns) {  // empty split: marked for the combine after the query transfer has landed
    if (w == 0 && lane < 16)
      a.part_ml[(int64_t(row) * a.H + h0 + lane) * a.n_split + j] = make_float2(-INFINITY, 0.f);
    wait_vmcnt<0>();
    return;
  }
  const int L = ctx - a.q_len + iq + 1;
  int kb1 = kb0 + a.split_blocks;
  const int lblk = (L + BLK - 1) / BLK;
  if (kb1 > lblk) kb1 = lblk;
  const int span = kb1 - kb0 - w;
  const int nwb = span > 0 ? (span + NW - 1) / NW : 0;

  // transfer of the wave's block i into ring stage i % NS: 10 full kilobytes, then 256 bytes (lanes
  // 16..63 of the last transfer re-read the block's start into the stage padding)
  auto issue = [&](int i) {
    const int phys = phys_of(i);
    const char* blk = unsigned(phys) < unsigned(a.num_blocks) ? cache + int64_t(phys) * kFp8Block : zero;
    const uint32_t dst = __builtin_amdgcn_readfirstlane(uint32_t(uintptr_t(ring + (i % NS) * kStage8)));
#pragma unroll
    for (int k = 0; k < 10; ++k) dma16(blk + 1024 * k + 16 * lane, dst + 1024 * k);
    dma16(blk + (lane < 16 ? 10240 : 0) + 16 * lane, dst + 10240);
  };

  const int pre = nwb < NS - 1 ? nwb : NS - 1;
  for (int i = 0; i < pre; ++i) issue(i);
  wait_blocks8(pre);  // the query transfers precede the blocks'
  lds_barrier();

  const int sc_off = 9216 * (r16 >> 3) + 128 * g + 16 * (r16 & 7);
  const int tr_off = 9216 * (g >> 1) + 64 * (g & 1) + 128 * ((r16 >> 1) & 1) + 16 * (r16 >> 2) + 8 * (r16 & 1);
  u32x4_t qreg[18];
  {
    const lds_u32x4_t* qp = (const lds_u32x4_t*)((lds_char_t*)q_mem + sc_off);
#pragma unroll
    for (int k = 0; k < 18; ++k) qreg[k] = qp[32 * k];
  }

  // conversion lane roles: token ct = lane % 16, granules c = lane / 16 + 4 e (e = 0..17) of the
  // bf16 tile (granule c of token t at chunk 9 (t / 8) + c / 8, slot 8 (c % 8) + t % 8)
  const int ct = lane & 15;
  const int cw_off = 9216 * (ct >> 3) + 16 * (ct & 7);       // + 1024 (c / 8) + 128 (c % 8)
  const int cr_off = kFp8Row * ct;                           // token ct's row in the fp8 stage

  f32x4_t acc[32];
#pragma unroll
  for (int jj = 0; jj < 32; ++jj) acc[jj] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  float m = -INFINITY, lsum = 0.f;

  for (int i = 0; i < nwb; ++i) {
    if (i + NS - 1 < nwb) issue(i + NS - 1);
    const int ahead = nwb - 1 - i < NS - 1 ? nwb - 1 - i : NS - 1;
    wait_blocks8(ahead);
    asm volatile("" ::: "memory");
    const int kb = kb0 + w + NW * i;
    lds_char_t* const st8 = ring + (i % NS) * kStage8;

    // fp8 stage -> bf16 tile (this wave's own); tokens past the visible range become zeros
    {
      const bool vis = kb * BLK + ct < L;
      const lds_char_t* src = st8 + cr_off;
#pragma unroll
      for (int e = 0; e < 18; ++e) {
        const int c = g + 4 * e;
        u32x4_t v;
        if (e < 16) {  // latent granule: 8 codes -> 8 bf16
          const u32x2_t cw = *(const __attribute__((address_space(3))) u32x2_t*)(src + 8 * c);
          v = u32x4_t{__builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(cw[0], 1.f, false)),
                      __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(cw[0], 1.f, true)),
                      __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(cw[1], 1.f, false)),
                      __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(cw[1], 1.f, true))};
        } else {       // rope granule: 8 bf16 as stored
          v = *(const lds_u32x4_t*)(src + DC + 16 * (c - 64));
        }
        if (!vis) v = u32x4_t{0u, 0u, 0u, 0u};
        *(__attribute__((address_space(3))) u32x4_t*)(tile + cw_off + 1024 * (c >> 3) + 128 * (c & 7)) = v;
      }
    }
    // group scales of this lane's tokens 4g + r (zero past the visible range, like their codes)
    f32x4_t scl[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      scl[r] = *(const __attribute__((address_space(3))) f32x4_t*)(st8 + kFp8Row * (4 * g + r) + DC + 2 * DR);
      if (kb * BLK + 4 * g + r >= L) scl[r] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    }
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // the tile is written before it is read

    // scores: four latent groups (MFMA k = 4G .. 4G+3) and the rope part (k = 16, 17) in separate
    // accumulators; lane holds tokens 4g + r of row r16
    const uint32_t tbase = uint32_t(uintptr_t(tile));
    uint32_t spa = tbase + uint32_t(sc_off);
    asm volatile("" : "+v"(spa));
    const lds_u32x4_t* sp = (const lds_u32x4_t*)uintptr_t(spa);
    constexpr int D = 4;
    u32x4_t rg[D];
#pragma unroll
    for (int k = 0; k < D; ++k) rg[k] = sp[32 * k];
    f32x4_t scg[5];
#pragma unroll
    for (int G = 0; G < 5; ++G) scg[G] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int k = 0; k < 18; ++k) {
      const u32x4_t x = rg[k % D];
      if (k + D < 18) rg[k % D] = sp[32 * (k + D)];
      scg[k >> 2] = mfma32v(x, qreg[k], scg[k >> 2]);
    }
    __builtin_amdgcn_sched_group_barrier(0x100, D, 0);
#pragma unroll
    for (int k = 0; k < 18 - D; ++k) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x008, D, 0);
    float sv[4];
    float mb = -INFINITY;
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      float s = scg[4][t];
#pragma unroll
      for (int G = 0; G < 4; ++G) s = fmaf(scl[t][G], scg[G][t], s);
      sv[t] = (kb * BLK + 4 * g + t < L) ? s : -INFINITY;
      mb = fmaxf(mb, sv[t]);
    }
    mb = fmaxf(mb, __shfl_xor(mb, 16, 64));
    mb = fmaxf(mb, __shfl_xor(mb, 32, 64));
    if (__any(mb > m + kMaxSlack)) {
      const float mn = fmaxf(m, mb);
      const float alpha = (m == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(m - mn);
      lsum *= alpha;
#pragma unroll
      for (int jj = 0; jj < 32; ++jj) acc[jj] *= alpha;
      m = mn;
    }
    float p[4];
#pragma unroll
    for (int t = 0; t < 4; ++t) p[t] = sv[t] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(sv[t] - m);
    lsum += (p[0] + p[1]) + (p[2] + p[3]);
    s16x4_t pb[4];  // P of the lane's tokens times their group-G scale, as the B operand
#pragma unroll
    for (int G = 0; G < 4; ++G)
      pb[G] = __builtin_bit_cast(s16x4_t, make_uint2(cvt_pk_bf16(p[0] * scl[0][G], p[1] * scl[1][G]),
                                                     cvt_pk_bf16(p[2] * scl[2][G], p[3] * scl[3][G])));

    // P.C: channel tile jj (group jj / 8) by transposed LDS read of the bf16 tile
    uint32_t tpa = tbase + uint32_t(tr_off);
    asm volatile("" : "+v"(tpa));
    lds_char_t* tp = (lds_char_t*)uintptr_t(tpa);
    constexpr int DT = 8;
    s16x4_t tv[DT];
#pragma unroll
    for (int jj = 0; jj < DT; ++jj) tv[jj] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)(tp + 256 * jj));
#pragma unroll
    for (int jj = 0; jj < 32; ++jj) {
      const s16x4_t av = tv[jj % DT];
      if (jj + DT < 32)
        tv[jj % DT] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)(tp + 256 * (jj + DT)));
      acc[jj] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(av, pb[jj >> 3], acc[jj], 0, 0, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x100, DT, 0);
#pragma unroll
    for (int jj = 0; jj < 32 - DT; ++jj) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x008, DT, 0);
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // tile and stage reads done before reuse
  }

  // merge of the two waves and the fp16 partial store, as in the bf16 kernel
  lsum += __shfl_xor(lsum, 16, 64);
  lsum += __shfl_xor(lsum, 32, 64);
  if (g == 0) {
    m_lds[w][r16] = m;
    l_lds[w][r16] = lsum;
  }
  __syncthreads();  // every wave's transfers have landed, the rings are free
  float M = -INFINITY;
#pragma unroll
  for (int ww = 0; ww < NW; ++ww) M = fmaxf(M, m_lds[ww][r16]);
  float Ltot = 0.f;
#pragma unroll
  for (int ww = 0; ww < NW; ++ww) {
    const float mw = m_lds[ww][r16];
    if (mw != -INFINITY) Ltot += __builtin_amdgcn_exp2f(mw - M) * l_lds[ww][r16];
  }
  const float sw = (m == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(m - M);
#pragma unroll
  for (int jj = 0; jj < 32; ++jj) acc[jj] *= sw;

  f32x4_t* slots = reinterpret_cast<f32x4_t*>(ring_mem);  // region r = tiles 16r..16r+15
  if (w == 0) {
#pragma unroll
    for (int t = 0; t < 16; ++t) slots[(16 + t) * 64 + lane] = acc[16 + t];
  } else {
#pragma unroll
    for (int t = 0; t < 16; ++t) slots[t * 64 + lane] = acc[t];
  }
  __syncthreads();
  f32x4_t fin[16];
  if (w == 0) {
#pragma unroll
    for (int t = 0; t < 16; ++t) fin[t] = acc[t] + slots[t * 64 + lane];
  } else {
#pragma unroll
    for (int t = 0; t < 16; ++t) fin[t] = slots[(16 + t) * 64 + lane] + acc[16 + t];
  }
  float mx = 0.f;
#pragma unroll
  for (int t = 0; t < 16; ++t)
#pragma unroll
    for (int e = 0; e < 4; ++e) mx = fmaxf(mx, fabsf(fin[t][e]));
  mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
  mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
  if (g == 0) x_lds[w][r16] = mx;
  __syncthreads();
  const float inv = Ltot > 0.f ? 1.f / Ltot : 0.f;
  const float down = fp16_fit_scale(fmaxf(x_lds[0][r16], x_lds[1][r16]) * inv);
  const float sc = inv * down;
  lds_char_t* const otile = (lds_char_t*)ring_mem + 32 * 64 * 16;
  auto put = [&](int jj, f32x4_t v) {
    v *= sc;
    const int G = 2 * jj + (g >> 1);
    *(lds_u32x2_t*)(otile + r16 * 1024 + 16 * (G ^ r16) + 8 * (g & 1)) =
        u32x2_t{cvt_pk_f16(v[0], v[1]), cvt_pk_f16(v[2], v[3])};
  };
#pragma unroll
  for (int t = 0; t < 16; ++t) put(16 * w + t, fin[t]);
  __syncthreads();
  const int64_t pidx = (int64_t(row) * a.H + h0 + r16) * a.n_split + j;
#pragma unroll
  for (int r = 8 * w; r < 8 * w + 8; ++r) {
    const int64_t pr = (int64_t(row) * a.H + h0 + r) * a.n_split + j;
    *reinterpret_cast<u32x4_t*>(a.part_o16 + pr * DC + 8 * lane) =
        *(const lds_u32x4_t*)(otile + r * 1024 + 16 * (lane ^ r));
  }
  if (w == 0 && g == 0) {
    a.part_ml[pidx] = make_float2(M, Ltot);
    a.part_scale[pidx] = 1.f / down;
  }
}

hipError_t launch_decode_fp8(const DecodeArgs& a, hipStream_t s) {
  const int grid = ((a.units + 7) >> 3) << 3;
  decode_fp8_kernel<2, 4><<<grid, 128, 0, s>>>(a);
  return hipGetLastError();
}

}  // namespace mla
