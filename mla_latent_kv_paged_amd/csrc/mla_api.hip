// Host side of libmla: argument validation, context ownership, workspace sizing, the split
// heuristic and the launch sequence of one decode step.  Every entry point is extern "C" and
// returns an mla_status; no exception crosses the boundary.
#include <algorithm>
#include <cmath>
#include <cstdlib>
#include <cstring>
#include <mutex>
#include <new>
#include <vector>

#include "mla_internal.h"

using namespace mla;

namespace mla {
thread_local LaunchEvents* t_launch_events = nullptr;
}  // namespace mla

// Decode scratch of mla_decode_noalloc: one static region per GPU, held by the loaded library until
// the process ends.  Host code never passes its name to a kernel (on the host the name is only a
// stand-in): the region's device address is looked up once per device, with that device current,
// and used from then on.
constexpr size_t kScratchBytes = size_t(64) << 20;
static __device__ __align__(256) char scratch[kScratchBytes];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// This device's address of the scratch region (the current device must be `dev`).
hipError_t scratch_address(int dev, void** out) {
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    const hipError_t e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return hipSuccess;
}
}  // namespace

namespace {

constexpr int kMaxSplit = 32;      // upper bound of splits per sequence (sizes the workspace)
constexpr int kProfRing = 1024;    // event pairs kept per kernel id while profiling

struct Prof {
  bool on = false;
  hipEvent_t ev[MLA_K_COUNT][kProfRing][2] = {};
  int64_t count[MLA_K_COUNT] = {};
  double total_ms[MLA_K_COUNT] = {};
  bool created = false;
};

}  // namespace

struct mla_ctx {
  mla_config cfg;
  bool bf16 = false;  // bf16 inputs, weights and outputs (MLA_BF16 and MLA_BF16_FP8)
  bool fp8 = false;   // FP8 cache rows (MLA_BF16_FP8)
  int device = 0;
  int cu_count = 256;
  float qscale = 0.f;
  void* W_uk = nullptr;
  void* W_ukT = nullptr;
  void* W_uv = nullptr;
  void* W_uvT = nullptr;
  void* zero_block = nullptr;
  double* gamma = nullptr;
  double2* rope = nullptr;
  void* qcat = nullptr;
  float* part_acc = nullptr;
  float2* part_ml = nullptr;
  float* part_scale = nullptr;
  int2* piece_tbl = nullptr;  // 32-row kernel: per stream (first piece id, piece count)
  int32_t max_wg32 = 0;       // 32-row kernel: most workgroups the partial buffer holds pieces for
  int32_t max_split = 1;
  int32_t forced_split_blocks = 0;
  int32_t forced_waves = 0;
  int32_t last_split_blocks = 0, last_n_split = 0, last_waves = 0;
  void* scratch = nullptr;  // this device's static scratch region (mla_decode_noalloc)
  // layer step (mla_layer_weights)
  int32_t hidden_dim = 0;     // 0: no layer attached
  int32_t layer_flags = 0;
  void* W1 = nullptr;         // [H*QW + ROW, D] bf16: q_proj rows, then kv_a_proj rows (times gamma_in)
  void* Wo = nullptr;         // [D, H*DV] bf16
  void* l_q = nullptr;        // [max_q_tokens, H, QW] bf16 queries
  float* l_ckv = nullptr;     // [max_q_tokens, ROW] fp32 [c_kv | k_pe] rows
  void* l_attn = nullptr;     // [max_q_tokens, H, DV] bf16 attention output
  float* l_part = nullptr;    // projection partial tiles (ProjArgs::part), sized for both projections
  float* l_ss = nullptr;      // their per-token sums of squares
  Prof prof;
};

namespace {

inline hipStream_t as_stream(void* s) { return static_cast<hipStream_t>(s); }

void ctx_release(mla_ctx* c) {
  if (!c) return;
  hipFree(c->W_uk);
  hipFree(c->W_ukT);
  hipFree(c->W_uv);
  hipFree(c->W_uvT);
  hipFree(c->zero_block);
  hipFree(c->gamma);
  hipFree(c->rope);
  hipFree(c->qcat);
  hipFree(c->part_acc);
  hipFree(c->part_ml);
  hipFree(c->part_scale);
  hipFree(c->piece_tbl);
  hipFree(c->W1);
  hipFree(c->Wo);
  hipFree(c->l_q);
  hipFree(c->l_ckv);
  hipFree(c->l_attn);
  hipFree(c->l_part);
  hipFree(c->l_ss);
  if (c->prof.created)
    for (int k = 0; k < MLA_K_COUNT; ++k)
      for (int i = 0; i < kProfRing; ++i) {
        hipEventDestroy(c->prof.ev[k][i][0]);
        hipEventDestroy(c->prof.ev[k][i][1]);
      }
  delete c;
}

// Accumulate the elapsed time of ring slot i of kernel k (waits for its events).
void prof_harvest(mla_ctx* c, int k, int64_t slot_count) {
  const int i = int(slot_count % kProfRing);
  float ms = 0.f;
  if (hipEventSynchronize(c->prof.ev[k][i][1]) == hipSuccess &&
      hipEventElapsedTime(&ms, c->prof.ev[k][i][0], c->prof.ev[k][i][1]) == hipSuccess)
    c->prof.total_ms[k] += ms;
}

// One profiled region: its launches carry the region's event pair (launch() in mla_internal.h), so
// the pair times the kernels themselves.  A region that launched nothing records both events here.
struct ProfScope {
  mla_ctx* c;
  int k;
  hipStream_t s;
  bool on;
  LaunchEvents le{};
  LaunchEvents* prev = nullptr;
  ProfScope(mla_ctx* c_, int k_, hipStream_t s_) : c(c_), k(k_), s(s_), on(c_->prof.on) {
    if (!on) return;
    const int64_t n = c->prof.count[k];
    if (n >= kProfRing) prof_harvest(c, k, n - kProfRing);  // slot about to be reused
    le = LaunchEvents{c->prof.ev[k][n % kProfRing][0], c->prof.ev[k][n % kProfRing][1], false};
    prev = t_launch_events;
    t_launch_events = &le;
  }
  ~ProfScope() {
    if (!on) return;
    t_launch_events = prev;
    const int64_t n = c->prof.count[k];
    if (!le.started) {
      hipEventRecord(le.start, s);
      hipEventRecord(le.stop, s);
    }
    c->prof.count[k] = n + 1;
  }
};

mla_status hip_status(hipError_t e) {
  if (e == hipSuccess) return MLA_OK;
  if (e == hipErrorOutOfMemory) return MLA_ENOMEM;
  return MLA_EHIP;
}

// Split size (in 16-token blocks) for a decode of `units` independent (sequence, row-tile) work
// items whose longest context spans max_blocks blocks.  The bf16 kernel holds one workgroup per
// CU, so the grid is sized to a whole number of workgroups per CU where possible
// (units * n_split ~ k * CUs); a split is capped so that a few long sequences in a ragged batch
// do not serialise the tail, and holds at least one block per wave.  With few units the splits
// are kept to at least sqrt(max_blocks) blocks: a split costs a workgroup's start-up and the
// combine one more partial per row to merge, against blocks that stream at a fraction of that
// each (at batch 1: about 0.5 us per block, 0.4 us per partial, 6 us per workgroup's start),
// so the step is shortest near sqrt(max_blocks) blocks per split.
int choose_split_blocks(const mla_ctx* c, int units, int max_blocks, int waves) {
  const int cus = c->cu_count;
  int n_target;
  if (units >= cus)
    n_target = 1;
  else
    n_target = cus / units;  // floor: units * n_target <= CUs, one round
  if (n_target < 1) n_target = 1;
  int sb = (max_blocks + n_target - 1) / n_target;
  int sq = 1;
  while (sq * sq < max_blocks) ++sq;
  if (sb < sq) sb = sq;
  const int cap = 128 * waves;
  if (sb > cap) sb = cap;
  if (sb < waves) sb = waves;
  return sb;
}

}  // namespace

namespace {
mla_status cache_write_args(const mla_ctx* ctx, const void* c_kv, int64_t c_kv_row_stride, const void* k_pe,
                            int64_t k_pe_row_stride, const int32_t* positions, const int32_t* slot_mapping,
                            int32_t num_tokens, void* kv_cache, int32_t num_blocks, CacheWriteArgs* a);
}  // namespace

extern "C" {

const char* mla_status_string(int32_t status) {
  switch (status) {
    case MLA_OK: return "MLA_OK";
    case MLA_EINVAL: return "MLA_EINVAL: invalid argument";
    case MLA_EUNSUPPORTED: return "MLA_EUNSUPPORTED: unsupported dimensions or dtype";
    case MLA_ENOMEM: return "MLA_ENOMEM: device allocation failed";
    case MLA_EHIP: return "MLA_EHIP: HIP runtime or launch failure";
    case MLA_ECAP: return "MLA_ECAP: size exceeds the context caps";
    default: return "unknown mla_status";
  }
}

mla_status mla_absorb_weights(const mla_config* cfg, const void* kv_b_proj_w, const void* kv_norm_gamma,
                              void* stream, mla_ctx** out) {
  if (out) *out = nullptr;
  if (!cfg || !kv_b_proj_w || !out) return MLA_EINVAL;
  if (cfg->dtype != MLA_F32 && cfg->dtype != MLA_BF16 && cfg->dtype != MLA_BF16_FP8) return MLA_EUNSUPPORTED;
  if (cfg->kv_lora_rank != DC || cfg->qk_rope_head_dim != DR || cfg->qk_nope_head_dim != DN ||
      cfg->v_head_dim != DV || cfg->block_size != BLK)
    return MLA_EUNSUPPORTED;
  if (cfg->num_heads <= 0 || cfg->num_heads % 16 != 0) return MLA_EUNSUPPORTED;
  if (cfg->max_q_tokens <= 0 || cfg->max_batch <= 0 || cfg->max_position < 0 || cfg->max_seq_len <= 0)
    return MLA_EINVAL;
  if (!(cfg->rms_eps >= 0.f) || !(cfg->rope_theta > 0.f)) return MLA_EINVAL;
  if (int64_t(cfg->max_q_tokens) * cfg->num_heads > (int64_t(1) << 24)) return MLA_ECAP;

  mla_ctx* c = new (std::nothrow) mla_ctx();
  if (!c) return MLA_ENOMEM;
  c->cfg = *cfg;
  c->bf16 = cfg->dtype != MLA_F32;
  c->fp8 = cfg->dtype == MLA_BF16_FP8;
  hipStream_t s = as_stream(stream);
  if (hipGetDevice(&c->device) != hipSuccess) {
    ctx_release(c);
    return MLA_EHIP;
  }
  // the static scratch region of this device (mla_decode_noalloc reports a failed lookup)
  if (scratch_address(c->device, &c->scratch) != hipSuccess) c->scratch = nullptr;

  hipDeviceProp_t prop;
  if (hipGetDeviceProperties(&prop, c->device) == hipSuccess && prop.multiProcessorCount > 0)
    c->cu_count = prop.multiProcessorCount;
  const double scale = cfg->softmax_scale > 0.f ? double(cfg->softmax_scale) : 1.0 / std::sqrt(double(DN + DR));
  c->qscale = float(scale * 1.4426950408889634);  // log2(e): scores in log2 units for exp2

  const int H = cfg->num_heads;
  const size_t esz = c->bf16 ? 2 : 4;
  const int max_blocks = (cfg->max_seq_len + BLK - 1) / BLK;
  // enough splits that a split never needs more than 128 blocks per wave at 2 waves per group
  const int need_split = (max_blocks + 255) / 256;
  c->max_split = max_blocks < kMaxSplit ? max_blocks : kMaxSplit;
  if (c->max_split < need_split) c->max_split = need_split;
  const size_t rows = size_t(cfg->max_q_tokens) * H;
  hipError_t e = hipSuccess;
  auto alloc = [&](void** p, size_t n) {
    if (e == hipSuccess) e = hipMalloc(p, n);
  };
  alloc(&c->W_uk, size_t(H) * DN * DC * esz);
  alloc(&c->W_ukT, size_t(H) * DC * DN * esz);
  alloc(&c->W_uv, size_t(H) * DV * DC * esz);
  alloc(&c->W_uvT, size_t(H) * DC * DV * esz);
  alloc(&c->zero_block, size_t(BLK) * ROW * esz);
  alloc(reinterpret_cast<void**>(&c->gamma), DC * sizeof(double));
  alloc(reinterpret_cast<void**>(&c->rope), size_t(cfg->max_position + 1) * NPAIR * sizeof(double2));
  alloc(&c->qcat, rows * ROW * esz);
  // partials: by split (rows x max_split) for the one-tile and fp32 kernels; by piece for the
  // 32-row kernel, at most (workgroups + streams) pieces of 32 T rows, i.e. at most
  // 128 * max_wg32 + rows rows (streams of a decode hold rows / (32 T) pieces' worth of rows)
  {
    // workgroups the 32-row kernel may need: a resident slot each, or enough that no range
    // exceeds kMt32MaxSteps steps at the caps (every stream at max_seq_len)
    const int64_t streams = std::max<int64_t>(1, int64_t(cfg->max_q_tokens) * H / 32);
    const int64_t steps_max = streams * ((max_blocks + 1) / 2 + kPieceCost);
    c->max_wg32 = int(std::max<int64_t>(2 * c->cu_count, (steps_max + kMt32MaxSteps - 1) / kMt32MaxSteps));
  }
  const size_t part_rows = std::max(rows * c->max_split, size_t(128) * c->max_wg32 + rows);
  alloc(reinterpret_cast<void**>(&c->part_acc), part_rows * DC * sizeof(float));
  alloc(reinterpret_cast<void**>(&c->part_ml), part_rows * sizeof(float2));
  alloc(reinterpret_cast<void**>(&c->part_scale), part_rows * sizeof(float));
  alloc(reinterpret_cast<void**>(&c->piece_tbl), (rows / 32 + 1) * sizeof(int2));
  if (e != hipSuccess) {
    ctx_release(c);
    return hip_status(e);
  }

  // gamma -> fp64 (exact upcast of the storage values)
  std::vector<double> g(DC, 1.0);
  if (kv_norm_gamma) {
    std::vector<uint8_t> raw(DC * esz);
    e = hipMemcpyAsync(raw.data(), kv_norm_gamma, DC * esz, hipMemcpyDeviceToHost, s);
    if (e == hipSuccess) e = hipStreamSynchronize(s);
    if (e != hipSuccess) {
      ctx_release(c);
      return hip_status(e);
    }
    for (int i = 0; i < DC; ++i) {
      if (c->bf16) {
        uint16_t bits;
        std::memcpy(&bits, raw.data() + 2 * i, 2);
        uint32_t u = uint32_t(bits) << 16;
        float f;
        std::memcpy(&f, &u, 4);
        g[i] = f;
      } else {
        float f;
        std::memcpy(&f, raw.data() + 4 * i, 4);
        g[i] = f;
      }
    }
  }
  // RoPE table: pair i at position p rotates by p * theta^(-2i/64); cos and sin in fp64
  std::vector<double2> rope(size_t(cfg->max_position + 1) * NPAIR);
  for (int i = 0; i < NPAIR; ++i) {
    const double inv_freq = std::pow(double(cfg->rope_theta), -2.0 * i / double(DR));
    for (int p = 0; p <= cfg->max_position; ++p) {
      const double ang = double(p) * inv_freq;
      rope[size_t(p) * NPAIR + i] = make_double2(std::cos(ang), std::sin(ang));
    }
  }
  e = hipMemsetAsync(c->zero_block, 0, size_t(BLK) * ROW * esz, s);
  if (e == hipSuccess) e = hipMemcpyAsync(c->gamma, g.data(), DC * sizeof(double), hipMemcpyHostToDevice, s);
  if (e == hipSuccess)
    e = hipMemcpyAsync(c->rope, rope.data(), rope.size() * sizeof(double2), hipMemcpyHostToDevice, s);
  if (e == hipSuccess) {
    AbsorbArgs aa{kv_b_proj_w, c->W_uk, c->W_ukT, c->W_uv, c->W_uvT, H};
    e = launch_absorb(c->bf16, aa, s);
  }
  if (e == hipSuccess) e = hipStreamSynchronize(s);
  if (e != hipSuccess) {
    ctx_release(c);
    return hip_status(e);
  }
  *out = c;
  return MLA_OK;
}

mla_status mla_cache_write(mla_ctx* ctx, const void* c_kv, int64_t c_kv_row_stride, const void* k_pe,
                           int64_t k_pe_row_stride, const int32_t* positions, const int32_t* slot_mapping,
                           int32_t num_tokens, void* kv_cache, int32_t num_blocks, void* stream) {
  CacheWriteArgs a;
  const mla_status st = cache_write_args(ctx, c_kv, c_kv_row_stride, k_pe, k_pe_row_stride, positions, slot_mapping,
                                         num_tokens, kv_cache, num_blocks, &a);
  if (st != MLA_OK || num_tokens == 0) return st;
  hipStream_t s = as_stream(stream);
  ProfScope ps(ctx, MLA_K_CACHE_WRITE, s);
  return hip_status(ctx->fp8 ? launch_cache_write_fp8(a, s) : launch_cache_write(ctx->bf16, a, s));
}

}  // extern "C"

namespace {
// The launch shape of one decode: kernel choice, split or partition, and the partial rows it writes.
struct DecodePlan {
  int t32 = 0;      // 32-row kernel: tiles per workgroup (0: a 16-row or the fp32 kernel)
  int n_rt = 0;     // row tiles per sequence (of 16 rows, or of 32 for the 32-row kernel)
  int waves = 0;
  int groups = 0;   // workgroups per (sequence, split): row tiles, or tile groups of the 32-row kernel
  int sb = 0, n_split = 0, n_wg = 0;
  int64_t part_rows = 0;  // partial rows written: by split, or by piece (32-row kernel)
  int64_t streams = 0;    // 32-row kernel: (sequence, tile group) pairs, one piece_tbl entry each
};

// The decode's scratch memory: [q_lat | q_pe'] rows, partial rows, their (m, l) and scales, and the
// piece table of the 32-row kernel.
struct DecodeWs {
  void* qcat;
  float* part_acc;  // fp32 partial rows; the bf16 kernels store fp16 rows in the same memory
  float2* part_ml;
  float* part_scale;
  int2* piece_tbl;
};

// Check a decode's host-visible arguments against the context's caps and choose its launch shape.
mla_status decode_plan(const mla_ctx* ctx, const void* q, int32_t batch, int32_t q_len, const void* kv_cache,
                       int32_t num_blocks, const int32_t* block_table, int32_t block_table_stride,
                       const int32_t* seq_lens, int32_t max_seq_len, const void* out, DecodePlan* pl) {
  if (!ctx || !q || !kv_cache || !block_table || !seq_lens || !out) return MLA_EINVAL;
  if (batch < 1 || q_len < 1 || num_blocks <= 0 || max_seq_len < q_len) return MLA_EINVAL;
  const mla_config& cf = ctx->cfg;
  if (batch > cf.max_batch || int64_t(batch) * q_len > cf.max_q_tokens || max_seq_len > cf.max_seq_len ||
      max_seq_len - 1 > cf.max_position)
    return MLA_ECAP;
  const int max_blocks = (max_seq_len + BLK - 1) / BLK;
  if (block_table_stride < max_blocks) return MLA_EINVAL;
  const int H = cf.num_heads;
  const int n_q = batch * q_len;

  DecodePlan p;
  const int n_rt16 = (H / 16) * q_len;  // row tiles of 16 per sequence (rows ordered query, head)
  // bf16 kernels by rows per sequence: a multiple of 32 -> 32-row tiles, T of them per workgroup
  // (each block read once per workgroup); otherwise the one-tile kernel, 16-row tiles in the grid
  const int n_rt32 = (H * q_len) % 32 == 0 ? H * q_len / 32 : 0;
  // (FP8 cache rows: the 16-row FP8 kernel for every shape)
  p.t32 = (ctx->bf16 && !ctx->fp8 && n_rt32 > 0) ? ((n_rt32 % 4 == 0) ? 4 : (n_rt32 % 2 == 0) ? 2 : 1) : 0;
  p.n_rt = p.t32 ? n_rt32 : n_rt16;
  p.waves = !ctx->bf16 ? 1
            : p.t32     ? p.t32
            : ctx->forced_waves > 0 ? ctx->forced_waves
            : ctx->fp8  ? 4
                        : 2;
  p.groups = p.t32 ? p.n_rt / p.t32 : p.n_rt;
  if (p.t32) {
    // balanced partition over one workgroup per resident slot (T = 4 fills a CU; T <= 2, two),
    // and enough workgroups that no range exceeds the block ids one workgroup stages in LDS
    p.n_wg = ctx->cu_count * (p.t32 == 4 ? 1 : 2);
    if (ctx->forced_split_blocks > 0) p.n_wg = ctx->forced_split_blocks;  // tuning: workgroup count
    const int64_t steps_max = int64_t(batch) * p.groups * ((max_blocks + 1) / 2 + kPieceCost);
    p.n_wg = int(std::max<int64_t>(p.n_wg, (steps_max + kMt32MaxSteps - 1) / kMt32MaxSteps));
    if (p.n_wg > ctx->max_wg32) return MLA_ECAP;
    // piece ids run up to (workgroups - 1) + (streams - 1); a piece holds 32 T rows
    p.streams = int64_t(batch) * p.groups;
    p.part_rows = (int64_t(p.n_wg) + p.streams) * 32 * p.t32;
  } else {
    p.sb = ctx->forced_split_blocks > 0 ? ctx->forced_split_blocks
                                        : choose_split_blocks(ctx, batch * p.groups, max_blocks, p.waves);
    const int min_sb = (max_blocks + ctx->max_split - 1) / ctx->max_split;  // workspace bound
    if (p.sb < min_sb) p.sb = min_sb;
    // the 16-row bf16 and FP8 kernels hold a wave's block ids in two registers: at most 128 blocks
    // per wave (max_split is sized so that min_sb never exceeds this at two or more waves); the
    // fp32 kernel reads its ids as it goes and has no such limit
    if (ctx->bf16 && p.sb > 128 * p.waves) p.sb = 128 * p.waves;
    if (p.sb > max_blocks) p.sb = max_blocks;
    p.n_split = (max_blocks + p.sb - 1) / p.sb;
    if (p.n_split > ctx->max_split) return MLA_ECAP;  // never past the partial workspace
    p.part_rows = int64_t(n_q) * H * p.n_split;
  }
  *pl = p;
  return MLA_OK;
}

// Bytes of scratch one decode of plan pl uses when its buffers are carved from one region (each
// buffer 256-byte aligned), and the carving itself when base is not null.
size_t decode_ws_carve(const mla_ctx* ctx, const DecodePlan& pl, int64_t n_q, char* base, DecodeWs* ws) {
  auto up = [](size_t x) { return (x + 255) & ~size_t(255); };
  const size_t esz = ctx->bf16 ? 2 : 4;
  const size_t H = size_t(ctx->cfg.num_heads);
  size_t off = 0;
  const size_t q_off = off;
  off += up(size_t(n_q) * H * ROW * esz);
  const size_t acc_off = off;
  off += up(size_t(pl.part_rows) * DC * esz);  // fp16 rows (bf16 kernels) or fp32 rows
  const size_t ml_off = off;
  off += up(size_t(pl.part_rows) * sizeof(float2));
  const size_t sc_off = off;
  off += up(size_t(pl.part_rows) * sizeof(float));
  const size_t pt_off = off;
  off += up(size_t(pl.streams + 1) * sizeof(int2));
  if (base && ws) {
    ws->qcat = base + q_off;
    ws->part_acc = reinterpret_cast<float*>(base + acc_off);
    ws->part_ml = reinterpret_cast<float2*>(base + ml_off);
    ws->part_scale = reinterpret_cast<float*>(base + sc_off);
    ws->piece_tbl = reinterpret_cast<int2*>(base + pt_off);
  }
  return off;
}

// mla_decode on the workspace ws with the launch shape pl; with cw, the cache write cw first
// (mla_decode_step): in the query absorption's launch for bf16 storage, else as its own launch
// before it
mla_status decode_launch(mla_ctx* ctx, const DecodePlan& pl, const DecodeWs& ws, const void* q, int32_t batch,
                         int32_t q_len, const void* kv_cache, int32_t num_blocks, const int32_t* block_table,
                         int32_t block_table_stride, const int32_t* seq_lens, int32_t max_seq_len, void* out,
                         hipStream_t s, const CacheWriteArgs* cw) {
  const mla_config& cf = ctx->cfg;
  const int H = cf.num_heads;
  const int n_q = batch * q_len;
  const int t32 = pl.t32;
  ctx->last_split_blocks = t32 ? 0 : pl.sb;
  ctx->last_n_split = t32 ? pl.n_wg : pl.n_split;
  ctx->last_waves = pl.waves;

  hipError_t e = hipSuccess;
  const bool fused = cw && cw->T > 0 && ctx->bf16;
  if (cw && cw->T > 0 && !fused) {
    ProfScope ps(ctx, MLA_K_CACHE_WRITE, s);
    e = ctx->fp8 ? launch_cache_write_fp8(*cw, s) : launch_cache_write(ctx->bf16, *cw, s);
  }
  if (e != hipSuccess) return hip_status(e);
  {
    QAbsorbArgs qa{q, ctx->W_uk, ctx->W_ukT, ctx->rope, seq_lens, q_len, n_q, H, max_seq_len, cf.max_position, ctx->qscale,
                   ws.qcat};
    ProfScope ps(ctx, fused ? MLA_K_PREP : MLA_K_Q_ABSORB, s);
    e = fused ? launch_decode_prep(qa, *cw, ctx->fp8, s) : launch_q_absorb(ctx->bf16, qa, s);
  }
  if (e != hipSuccess) return hip_status(e);
  {
    DecodeArgs da{batch,   kv_cache,    ctx->zero_block, num_blocks,  block_table,
                  block_table_stride,   seq_lens,        max_seq_len, q_len,
                  H,       ws.qcat,     ws.part_acc,     reinterpret_cast<uint16_t*>(ws.part_acc),
                  ws.part_ml,           ws.part_scale,   pl.sb,       pl.n_split,
                  pl.n_rt, t32 ? pl.n_wg : batch * pl.n_split * pl.groups,  ws.piece_tbl};
    ProfScope ps(ctx, MLA_K_DECODE, s);
    e = t32 ? launch_decode_mt32(da, t32, s)
            : ctx->fp8 ? launch_decode_fp8(da, pl.waves, s) : launch_decode(ctx->bf16, da, pl.waves, s);
  }
  if (e != hipSuccess) return hip_status(e);
  {
    // output channels split over 4 workgroups only when the (head, 16 rows) grid is small
    const int v_parts = int64_t(H) * ((n_q + 15) / 16) >= 2 * ctx->cu_count ? 1 : 4;
    // 64 rows per workgroup (W_uv read once per 64 rows) once that alone gives every CU a workgroup
    const int rows_wg = int64_t(H) * ((n_q + 63) / 64) >= ctx->cu_count ? 64 : 16;
    CombineArgs ca{ws.part_acc, reinterpret_cast<const uint16_t*>(ws.part_acc), ws.part_ml, ws.part_scale, seq_lens,
                   max_seq_len, q_len, n_q, H, pl.sb, pl.n_split, ctx->W_uv, ctx->W_uvT, out,
                   t32 ? ws.piece_tbl : nullptr, 32 * t32, t32 ? pl.n_rt / t32 : 0, v_parts, rows_wg};
    ProfScope ps(ctx, MLA_K_COMBINE, s);
    e = launch_combine(ctx->bf16, ca, s);
  }
  return hip_status(e);
}

// mla_decode (and mla_decode_step with cw) on the context's own workspace
mla_status decode_impl(mla_ctx* ctx, const void* q, int32_t batch, int32_t q_len, const void* kv_cache,
                       int32_t num_blocks, const int32_t* block_table, int32_t block_table_stride,
                       const int32_t* seq_lens, int32_t max_seq_len, void* out, hipStream_t s,
                       const CacheWriteArgs* cw) {
  DecodePlan pl;
  const mla_status st = decode_plan(ctx, q, batch, q_len, kv_cache, num_blocks, block_table, block_table_stride,
                                    seq_lens, max_seq_len, out, &pl);
  if (st != MLA_OK) return st;
  const DecodeWs ws{ctx->qcat, ctx->part_acc, ctx->part_ml, ctx->part_scale, ctx->piece_tbl};
  return decode_launch(ctx, pl, ws, q, batch, q_len, kv_cache, num_blocks, block_table, block_table_stride, seq_lens,
                       max_seq_len, out, s, cw);
}

// the arguments of a cache write, checked as mla_cache_write checks them
mla_status cache_write_args(const mla_ctx* ctx, const void* c_kv, int64_t c_kv_row_stride, const void* k_pe,
                            int64_t k_pe_row_stride, const int32_t* positions, const int32_t* slot_mapping,
                            int32_t num_tokens, void* kv_cache, int32_t num_blocks, CacheWriteArgs* a) {
  if (!ctx || num_tokens < 0) return MLA_EINVAL;
  if (num_tokens > 0 && (!c_kv || !k_pe || !positions || !slot_mapping || !kv_cache || num_blocks <= 0))
    return MLA_EINVAL;
  if (num_tokens > 0 && (c_kv_row_stride < DC || k_pe_row_stride < DR)) return MLA_EINVAL;
  *a = CacheWriteArgs{c_kv, c_kv_row_stride, k_pe, k_pe_row_stride, positions, slot_mapping, num_tokens,
                      kv_cache, int64_t(num_blocks) * BLK, ctx->gamma, ctx->rope, ctx->cfg.max_position,
                      double(ctx->cfg.rms_eps)};
  return MLA_OK;
}
}  // namespace

extern "C" {

mla_status mla_decode(mla_ctx* ctx, const void* q, int32_t batch, int32_t q_len, const void* kv_cache,
                      int32_t num_blocks, const int32_t* block_table, int32_t block_table_stride,
                      const int32_t* seq_lens, int32_t max_seq_len, void* out, void* stream) {
  return decode_impl(ctx, q, batch, q_len, kv_cache, num_blocks, block_table, block_table_stride, seq_lens,
                     max_seq_len, out, as_stream(stream), nullptr);
}

mla_status mla_decode_step(mla_ctx* ctx, const void* c_kv, int64_t c_kv_row_stride, const void* k_pe,
                           int64_t k_pe_row_stride, const int32_t* positions, const int32_t* slot_mapping,
                           int32_t num_tokens, const void* q, int32_t batch, int32_t q_len, void* kv_cache,
                           int32_t num_blocks, const int32_t* block_table, int32_t block_table_stride,
                           const int32_t* seq_lens, int32_t max_seq_len, void* out, void* stream) {
  CacheWriteArgs cw;
  const mla_status st = cache_write_args(ctx, c_kv, c_kv_row_stride, k_pe, k_pe_row_stride, positions, slot_mapping,
                                         num_tokens, kv_cache, num_blocks, &cw);
  if (st != MLA_OK) return st;
  return decode_impl(ctx, q, batch, q_len, kv_cache, num_blocks, block_table, block_table_stride, seq_lens,
                     max_seq_len, out, as_stream(stream), &cw);
}

mla_status mla_decode_noalloc(mla_ctx* ctx, const void* q, int32_t batch, int32_t q_len, const void* kv_cache,
                              int32_t num_blocks, const int32_t* block_table, int32_t block_table_stride,
                              const int32_t* seq_lens, int32_t max_seq_len, void* out, void* stream) {
  DecodePlan pl;
  const mla_status st = decode_plan(ctx, q, batch, q_len, kv_cache, num_blocks, block_table, block_table_stride,
                                    seq_lens, max_seq_len, out, &pl);
  if (st != MLA_OK) return st;
  if (!ctx->scratch) return MLA_EHIP;  // the scratch lookup failed when the context was made
  const int64_t n_q = int64_t(batch) * q_len;
  if (decode_ws_carve(ctx, pl, n_q, nullptr, nullptr) > kScratchBytes) return MLA_ECAP;
  DecodeWs ws;
  decode_ws_carve(ctx, pl, n_q, static_cast<char*>(ctx->scratch), &ws);
  return decode_launch(ctx, pl, ws, q, batch, q_len, kv_cache, num_blocks, block_table, block_table_stride, seq_lens,
                       max_seq_len, out, as_stream(stream), nullptr);
}

mla_status mla_layer_weights(mla_ctx* ctx, int32_t hidden_dim, const void* q_proj_w, const void* kv_a_proj_w,
                             const void* o_proj_w, const void* input_norm_gamma, int32_t flags, void* stream) {
  if (!ctx || !q_proj_w || !kv_a_proj_w || !o_proj_w) return MLA_EINVAL;
  if (flags & ~(MLA_LAYER_INPUT_NORM | MLA_LAYER_RESIDUAL)) return MLA_EINVAL;
  if (!ctx->bf16 || hidden_dim <= 0 || hidden_dim % kProjChunk != 0) return MLA_EUNSUPPORTED;
  const int H = ctx->cfg.num_heads;
  const int64_t n1 = int64_t(H) * QW + ROW;
  const size_t mq = size_t(ctx->cfg.max_q_tokens);
  auto release = [&]() {
    hipFree(ctx->W1);
    hipFree(ctx->Wo);
    hipFree(ctx->l_q);
    hipFree(ctx->l_ckv);
    hipFree(ctx->l_attn);
    hipFree(ctx->l_part);
    hipFree(ctx->l_ss);
    ctx->W1 = ctx->Wo = ctx->l_q = ctx->l_attn = nullptr;
    ctx->l_ckv = ctx->l_part = ctx->l_ss = nullptr;
    ctx->hidden_dim = 0;
  };
  release();  // a second call replaces the first
  // projection workspace: both projections' output tiles of 64 and K chunks, for m tiles of 64 tokens
  const size_t m_tiles = (mq + 63) / 64;
  const size_t tiles_qkv = size_t(n1 / 64) * (hidden_dim / kProjChunk);
  const size_t tiles_o = size_t(hidden_dim / 64) * (H * DV / kProjChunk);
  const size_t tiles = std::max(tiles_qkv, tiles_o);
  const size_t chunks = std::max<size_t>(hidden_dim, size_t(H) * DV) / kProjChunk;
  hipError_t e = hipSuccess;
  auto alloc = [&](void** p, size_t n) {
    if (e == hipSuccess) e = hipMalloc(p, n);
  };
  alloc(&ctx->W1, size_t(n1) * hidden_dim * 2);
  alloc(&ctx->Wo, size_t(hidden_dim) * H * DV * 2);
  alloc(&ctx->l_q, mq * H * QW * 2);
  alloc(reinterpret_cast<void**>(&ctx->l_ckv), mq * ROW * sizeof(float));
  alloc(&ctx->l_attn, mq * H * DV * 2);
  alloc(reinterpret_cast<void**>(&ctx->l_part), m_tiles * tiles * 64 * 64 * sizeof(float));
  alloc(reinterpret_cast<void**>(&ctx->l_ss), m_tiles * chunks * 64 * sizeof(float));
  hipStream_t s = as_stream(stream);
  const void* g = (flags & MLA_LAYER_INPUT_NORM) ? input_norm_gamma : nullptr;
  if (e == hipSuccess) e = launch_layer_pack(q_proj_w, g, ctx->W1, int64_t(H) * QW, hidden_dim, s);
  if (e == hipSuccess)
    e = launch_layer_pack(kv_a_proj_w, g, static_cast<uint16_t*>(ctx->W1) + int64_t(H) * QW * hidden_dim, ROW,
                          hidden_dim, s);
  if (e == hipSuccess) e = launch_layer_pack(o_proj_w, nullptr, ctx->Wo, hidden_dim, H * DV, s);
  if (e == hipSuccess) e = hipStreamSynchronize(s);
  if (e != hipSuccess) {
    release();
    return hip_status(e);
  }
  ctx->hidden_dim = hidden_dim;
  ctx->layer_flags = flags;
  return MLA_OK;
}

mla_status mla_layer_decode_step(mla_ctx* ctx, const void* hidden, const int32_t* positions,
                                 const int32_t* slot_mapping, int32_t batch, int32_t q_len, void* kv_cache,
                                 int32_t num_blocks, const int32_t* block_table, int32_t block_table_stride,
                                 const int32_t* seq_lens, int32_t max_seq_len, void* out, void* stream) {
  if (!ctx || !ctx->hidden_dim || !hidden || !positions || !slot_mapping || !out) return MLA_EINVAL;
  DecodePlan pl;
  mla_status st = decode_plan(ctx, ctx->l_q, batch, q_len, kv_cache, num_blocks, block_table, block_table_stride,
                              seq_lens, max_seq_len, ctx->l_attn, &pl);
  if (st != MLA_OK) return st;
  const int H = ctx->cfg.num_heads;
  const int n_q = batch * q_len;
  const int D = ctx->hidden_dim;
  CacheWriteArgs cw;
  st = cache_write_args(ctx, ctx->l_ckv, ROW, ctx->l_ckv + DC, ROW, positions, slot_mapping, n_q, kv_cache,
                        num_blocks, &cw);
  if (st != MLA_OK) return st;
  cw.in_f32 = 1;
  hipStream_t s = as_stream(stream);
  hipError_t e;
  {
    ProjArgs pa{};
    pa.X = static_cast<const uint16_t*>(hidden);
    pa.x_stride = D;
    pa.W = static_cast<const uint16_t*>(ctx->W1);
    pa.M = n_q;
    pa.N = H * QW + ROW;
    pa.K = D;
    pa.norm = (ctx->layer_flags & MLA_LAYER_INPUT_NORM) ? 1 : 0;
    pa.eps = ctx->cfg.rms_eps;
    pa.mode = 0;
    pa.n_split = H * QW;
    pa.y0 = static_cast<uint16_t*>(ctx->l_q);
    pa.y1 = ctx->l_ckv;
    pa.part = ctx->l_part;
    pa.ss_part = ctx->l_ss;
    ProfScope ps(ctx, MLA_K_LAYER_QKV, s);
    e = launch_proj_gemm(pa, s);
  }
  if (e != hipSuccess) return hip_status(e);
  const DecodeWs ws{ctx->qcat, ctx->part_acc, ctx->part_ml, ctx->part_scale, ctx->piece_tbl};
  st = decode_launch(ctx, pl, ws, ctx->l_q, batch, q_len, kv_cache, num_blocks, block_table, block_table_stride,
                     seq_lens, max_seq_len, ctx->l_attn, s, &cw);
  if (st != MLA_OK) return st;
  {
    ProjArgs pa{};
    pa.X = static_cast<const uint16_t*>(ctx->l_attn);
    pa.x_stride = int64_t(H) * DV;
    pa.W = static_cast<const uint16_t*>(ctx->Wo);
    pa.M = n_q;
    pa.N = D;
    pa.K = H * DV;
    pa.mode = 1;
    pa.R = (ctx->layer_flags & MLA_LAYER_RESIDUAL) ? static_cast<const uint16_t*>(hidden) : nullptr;
    pa.out = static_cast<uint16_t*>(out);
    pa.part = ctx->l_part;
    pa.ss_part = ctx->l_ss;
    ProfScope ps(ctx, MLA_K_LAYER_O, s);
    e = launch_proj_gemm(pa, s);
  }
  return hip_status(e);
}

namespace {
int64_t prefill_tpad(int32_t max_seq_len) {  // a whole number of expansion workgroups
  return (int64_t(max_seq_len) + kPrefillTokens - 1) / kPrefillTokens * kPrefillTokens;
}
}  // namespace

mla_status mla_prefill_workspace_size(const mla_ctx* ctx, int32_t batch, int32_t total_q, int32_t max_seq_len,
                                      size_t* bytes) {
  if (!ctx || !bytes || batch < 1 || total_q < 1 || max_seq_len < 1) return MLA_EINVAL;
  const int64_t kv = int64_t(batch) * ctx->cfg.num_heads * prefill_tpad(max_seq_len) * (DN + DR + DV) * 2;
  const int64_t qr = int64_t(total_q) * ctx->cfg.num_heads * DR * 2;  // the rotated q_pe
  const int64_t lat = ctx->fp8 ? int64_t(batch) * prefill_tpad(max_seq_len) * ROW * 2 : 0;  // dequantised rows
  *bytes = size_t(kv + qr + lat);
  return MLA_OK;
}

mla_status mla_prefill(mla_ctx* ctx, const void* q, const int32_t* cu_q_lens, int32_t batch, int32_t total_q,
                       int32_t max_q_len, const void* kv_cache, int32_t num_blocks, const int32_t* block_table,
                       int32_t block_table_stride, const int32_t* seq_lens, int32_t max_seq_len, void* workspace,
                       size_t workspace_bytes, void* out, void* stream) {
  if (!ctx || !q || !cu_q_lens || !kv_cache || !block_table || !seq_lens || !workspace || !out) return MLA_EINVAL;
  if (batch < 1 || total_q < 1 || max_q_len < 1 || num_blocks <= 0 || max_seq_len < max_q_len) return MLA_EINVAL;
  if (!ctx->bf16) return MLA_EUNSUPPORTED;
  const mla_config& cf = ctx->cfg;
  if (max_seq_len - 1 > cf.max_position) return MLA_ECAP;
  const int max_blocks = (max_seq_len + BLK - 1) / BLK;
  if (block_table_stride < max_blocks) return MLA_EINVAL;
  size_t need = 0;
  mla_prefill_workspace_size(ctx, batch, total_q, max_seq_len, &need);
  if (workspace_bytes < need) return MLA_EINVAL;
  hipStream_t s = as_stream(stream);
  char* ws = static_cast<char*>(workspace);
  PrefillArgs pa{};
  pa.batch = batch;
  pa.H = cf.num_heads;
  pa.q = q;
  pa.cu_q_lens = cu_q_lens;
  pa.total_q = total_q;
  pa.max_q_len = max_q_len;
  pa.cache = kv_cache;
  pa.zero_block = ctx->zero_block;
  pa.num_blocks = num_blocks;
  pa.block_table = block_table;
  pa.bt_stride = block_table_stride;
  pa.seq_lens = seq_lens;
  pa.max_seq_len = max_seq_len;
  pa.max_position = cf.max_position;
  pa.t_pad = int32_t(prefill_tpad(max_seq_len));
  pa.rope = ctx->rope;
  pa.qscale = ctx->qscale;
  pa.W_uk = static_cast<const uint16_t*>(ctx->W_uk);
  pa.W_uv = static_cast<const uint16_t*>(ctx->W_uv);
  pa.kv = reinterpret_cast<uint16_t*>(ws);
  pa.qpe = reinterpret_cast<uint16_t*>(ws + int64_t(batch) * cf.num_heads * prefill_tpad(max_seq_len) * (DN + DR + DV) * 2);
  pa.lat = ctx->fp8 ? pa.qpe + int64_t(total_q) * cf.num_heads * DR : nullptr;
  pa.out = out;
  hipError_t e;
  {
    ProfScope ps(ctx, MLA_K_PF_EXPAND, s);
    e = launch_prefill_expand(pa, ctx->fp8, s);
  }
  if (e != hipSuccess) return hip_status(e);
  {
    ProfScope ps(ctx, MLA_K_PF_ATTN, s);  // the rotation of q_pe and the attention
    e = launch_prefill_qprep(pa, s);
    if (e == hipSuccess) e = launch_prefill_attn(pa, s);
  }
  return hip_status(e);
}

void mla_free(mla_ctx* ctx) {
  if (!ctx) return;
  hipDeviceSynchronize();
  ctx_release(ctx);
}

mla_status mla_ceiling_read(const void* src, int64_t bytes, void* sink, int64_t sink_bytes, void* stream) {
  constexpr int kGrid = 1024;
  if (!src || !sink || bytes <= 0 || bytes % 16 != 0 || sink_bytes < int64_t(kGrid) * 256 * 4) return MLA_EINVAL;
  return hip_status(launch_stream_read(src, bytes, static_cast<uint32_t*>(sink), kGrid, as_stream(stream)));
}

mla_status mla_ceiling_mfma(int32_t shape, int32_t iterations, void* sink, int64_t sink_bytes, double* flops,
                            void* stream) {
  if (!sink || (shape != 0 && shape != 1) || iterations < 1 || iterations > (1 << 20) ||
      sink_bytes < int64_t(kMfmaLoopGrid) * 256 * 4)
    return MLA_EINVAL;
  // eight 16x16x32 or four 32x32x16 MFMAs per wave and round: 2 x 16 x 16 x 32 x 8 flops either way
  if (flops) *flops = double(kMfmaLoopGrid) * 4 * double(iterations) * kMfmaChains * (2.0 * 16 * 16 * 32);
  return hip_status(
      launch_mfma_loop(shape, iterations, static_cast<uint32_t*>(sink), kMfmaLoopGrid, as_stream(stream)));
}

mla_status mla_ceiling_gather(mla_ctx* ctx, int32_t batch, int32_t q_len, const void* kv_cache, int32_t num_blocks,
                              const int32_t* block_table, int32_t block_table_stride, const int32_t* seq_lens,
                              int32_t max_seq_len, void* sink, int64_t sink_bytes, void* stream) {
  if (!sink) return MLA_EINVAL;
  DecodePlan pl;
  // the decode's own plan (its q and out pointers are not read: the sink stands in for both)
  const mla_status st = decode_plan(ctx, sink, batch, q_len, kv_cache, num_blocks, block_table, block_table_stride,
                                    seq_lens, max_seq_len, sink, &pl);
  if (st != MLA_OK) return st;
  if (!ctx->bf16 || ctx->fp8 || pl.t32 != 0 || pl.waves != 2) return MLA_EUNSUPPORTED;
  const int units = batch * pl.n_split * pl.groups;
  const int64_t grid = (int64_t(units) + 7) / 8 * 8;
  if (sink_bytes < grid * 128 * 4) return MLA_EINVAL;
  DecodeArgs da{};
  da.batch = batch;
  da.cache = kv_cache;
  da.zero_block = ctx->zero_block;
  da.num_blocks = num_blocks;
  da.block_table = block_table;
  da.bt_stride = block_table_stride;
  da.seq_lens = seq_lens;
  da.max_seq_len = max_seq_len;
  da.q_len = q_len;
  da.H = ctx->cfg.num_heads;
  da.split_blocks = pl.sb;
  da.n_split = pl.n_split;
  da.n_rt = pl.n_rt;
  da.units = units;
  return hip_status(launch_gather_dma(da, static_cast<uint32_t*>(sink), as_stream(stream)));
}

mla_status mla_set_decode_tuning(mla_ctx* ctx, int32_t split_blocks, int32_t waves_per_group) {
  if (!ctx || split_blocks < 0) return MLA_EINVAL;
  // 2 or 4 for the 16-row kernels (bf16 and FP8 rows)
  if (waves_per_group != 0 && waves_per_group != 2 && waves_per_group != 4) return MLA_EINVAL;
  ctx->forced_split_blocks = split_blocks;
  ctx->forced_waves = waves_per_group;
  return MLA_OK;
}

mla_status mla_last_decode_shape(const mla_ctx* ctx, int32_t* split_blocks, int32_t* n_split,
                                 int32_t* waves_per_group) {
  if (!ctx) return MLA_EINVAL;
  if (split_blocks) *split_blocks = ctx->last_split_blocks;
  if (n_split) *n_split = ctx->last_n_split;
  if (waves_per_group) *waves_per_group = ctx->last_waves;
  return MLA_OK;
}

mla_status mla_profile_enable(mla_ctx* ctx, int32_t enable) {
  if (!ctx) return MLA_EINVAL;
  if (enable && !ctx->prof.created) {
    for (int k = 0; k < MLA_K_COUNT; ++k)
      for (int i = 0; i < kProfRing; ++i)
        for (int h = 0; h < 2; ++h)
          if (hipEventCreate(&ctx->prof.ev[k][i][h]) != hipSuccess) return MLA_EHIP;
    ctx->prof.created = true;
  }
  if (enable)
    for (int k = 0; k < MLA_K_COUNT; ++k) {
      ctx->prof.count[k] = 0;
      ctx->prof.total_ms[k] = 0.0;
    }
  ctx->prof.on = enable != 0;
  return MLA_OK;
}

mla_status mla_profile_read(mla_ctx* ctx, int32_t kernel_id, double* total_ms, int64_t* launches) {
  if (!ctx || kernel_id < 0 || kernel_id >= MLA_K_COUNT) return MLA_EINVAL;
  const int64_t n = ctx->prof.count[kernel_id];
  const int64_t first = n > kProfRing ? n - kProfRing : 0;
  double extra = 0.0;
  const double before = ctx->prof.total_ms[kernel_id];
  for (int64_t i = first; i < n; ++i) prof_harvest(ctx, kernel_id, i);
  extra = ctx->prof.total_ms[kernel_id] - before;
  // the harvested slots stay in the ring: undo so that a second read does not double count
  ctx->prof.total_ms[kernel_id] = before;
  if (total_ms) *total_ms = before + extra;
  if (launches) *launches = n;
  return MLA_OK;
}

mla_status mla_profile_samples(mla_ctx* ctx, int32_t kernel_id, float* ms, int32_t max, int32_t* n_out) {
  if (n_out) *n_out = 0;
  if (!ctx || kernel_id < 0 || kernel_id >= MLA_K_COUNT || max < 0 || (!ms && max > 0)) return MLA_EINVAL;
  const int64_t n = ctx->prof.count[kernel_id];
  int64_t first = n > kProfRing ? n - kProfRing : 0;
  if (n - first > max) first = n - max;
  int32_t m = 0;
  for (int64_t i = first; i < n; ++i) {
    const int slot = int(i % kProfRing);
    float t = 0.f;
    if (hipEventSynchronize(ctx->prof.ev[kernel_id][slot][1]) != hipSuccess ||
        hipEventElapsedTime(&t, ctx->prof.ev[kernel_id][slot][0], ctx->prof.ev[kernel_id][slot][1]) != hipSuccess)
      return MLA_EHIP;
    ms[m++] = t;
  }
  if (n_out) *n_out = m;
  return MLA_OK;
}

}  // extern "C"
