// Split-K GQA decode attention, MFMA path for 65..128 query rows per launch
// with pages of a multiple of 32 tokens (cascade prefix pass: 24-ai.news
// TokenSpeed article, optimisation list, hybrid prefix caching).  The body
// and its gfx950 mapping are in attn_mfma128_body.h.
#include "attn_mfma128_body.h"

namespace had {
namespace {

// one workgroup per CU (the LDS stage buffers take most of it)
template <int D>
__global__ __launch_bounds__(64 * kM128Waves, 1) void attn_mfma128_kernel(ValuArgs a) {
  mfma128_partial<D>(a, blockIdx.x, blockIdx.y, blockIdx.z);
}

}  // namespace

hipError_t launch_attn_mfma128(const ValuArgs& a, int head_dim, dim3 grid, hipStream_t stream) {
  if (a.page_size % 32 != 0) return hipErrorInvalidValue;  // (rows row_base .. row_base + 127 of the launch)
  const dim3 blk(64 * kM128Waves);
  switch (head_dim) {
    case 64: hipLaunchKernelGGL((attn_mfma128_kernel<64>), grid, blk, 0, stream, a); break;
    case 128: hipLaunchKernelGGL((attn_mfma128_kernel<128>), grid, blk, 0, stream, a); break;
    case 256: hipLaunchKernelGGL((attn_mfma128_kernel<256>), grid, blk, 0, stream, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace had
