// Split-K GQA decode attention, MFMA path with K and V loaded straight into
// LDS, for pages of a multiple of 32 tokens: 65..128 query rows per launch
// (cascade prefix pass: 24-ai.news TokenSpeed article, optimisation list,
// hybrid prefix caching) and, at head_dim 128 or 256, 16..64 rows (the
// verify of a speculative draft: zubnet.ai TokenSpeed article, second
// paragraph).  The body and its gfx950 mapping are in attn_mfma128_body.h.
#include "attn_mfma128_body.h"

namespace had {
namespace {

// one workgroup per CU (the LDS stage buffers take most of it)
template <int D, int DH>
__global__ __launch_bounds__(64 * kM128Waves, 1) void attn_mfma128_kernel(ValuArgs a) {
  mfma128_partial<D, DH>(a, blockIdx.x, blockIdx.y, blockIdx.z);
}

}  // namespace

hipError_t launch_attn_mfma128(const ValuArgs& a, int head_dim, int dh, dim3 grid, hipStream_t stream) {
  // (rows row_base .. row_base + 128 / dh - 1 of the launch)
  if (a.page_size % 32 != 0 || (dh != 1 && dh != 2) || (dh == 2 && head_dim < 128)) return hipErrorInvalidValue;
  const dim3 blk(64 * kM128Waves);
  switch (head_dim * 2 + dh - 1) {
    case 128: hipLaunchKernelGGL((attn_mfma128_kernel<64, 1>), grid, blk, 0, stream, a); break;
    case 256: hipLaunchKernelGGL((attn_mfma128_kernel<128, 1>), grid, blk, 0, stream, a); break;
    case 257: hipLaunchKernelGGL((attn_mfma128_kernel<128, 2>), grid, blk, 0, stream, a); break;
    case 512: hipLaunchKernelGGL((attn_mfma128_kernel<256, 1>), grid, blk, 0, stream, a); break;
    case 513: hipLaunchKernelGGL((attn_mfma128_kernel<256, 2>), grid, blk, 0, stream, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace had
