// S0 -- weight absorption split (mini-infer 17 "MLA Attention：从 KV Cache 压缩到矩阵吸收",
// 版本 3 _build_absorbed): kv_b_proj viewed as (H, DN + DV, DC); per head the DN "nope" rows are
// W_uk and the DV "value" rows are W_uv.  Pure data movement, no arithmetic; each factor is kept
// in the two layouts its consumers read:
//   W_uk [H, DN, DC]  rows h*(DN+DV) + n, DC contiguous        (fp32 query kernel)
//   W_ukT[H, DC, DN]  its transpose, DN contiguous             (MFMA query kernel: K = DN)
//   W_uv [H, DV, DC]  rows h*(DN+DV) + DN + v, DC contiguous   (MFMA output kernel: K = DC)
//   W_uvT[H, DC, DV]  its transpose, DV contiguous             (fp32 output kernel)
#include "mla_internal.h"

namespace mla {

template <typename T>
__global__ __launch_bounds__(256) void absorb_kernel(AbsorbArgs a) {
  const T* src = static_cast<const T*>(a.kv_b_proj);
  T* wuk = static_cast<T*>(a.W_uk);
  T* wukt = static_cast<T*>(a.W_ukT);
  T* wuv = static_cast<T*>(a.W_uv);
  T* wuvt = static_cast<T*>(a.W_uvT);
  const int64_t total = int64_t(a.H) * (DN + DV) * DC;
  for (int64_t i = int64_t(blockIdx.x) * blockDim.x + threadIdx.x; i < total; i += int64_t(gridDim.x) * blockDim.x) {
    const int c = int(i % DC);
    const int64_t rowi = i / DC;
    const int h = int(rowi / (DN + DV));
    const int r = int(rowi % (DN + DV));
    if (r < DN) {
      wuk[(int64_t(h) * DN + r) * DC + c] = src[i];
      wukt[(int64_t(h) * DC + c) * DN + r] = src[i];
    } else {
      wuv[(int64_t(h) * DV + (r - DN)) * DC + c] = src[i];
      wuvt[(int64_t(h) * DC + c) * DV + (r - DN)] = src[i];
    }
  }
}

hipError_t launch_absorb(bool bf16, const AbsorbArgs& a, hipStream_t s) {
  const int64_t total = int64_t(a.H) * (DN + DV) * DC;
  const int grid = int((total + 255) / 256 < 65536 ? (total + 255) / 256 : 65536);
  if (bf16)
    launch(absorb_kernel<uint16_t>, dim3(grid), dim3(256), 0, s, a);
  else
    launch(absorb_kernel<float>, dim3(grid), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace mla
