// Split-K GQA decode attention, MFMA path with K and V loaded straight into
// LDS, for pages of a multiple of 32 tokens: 65..128 query rows per launch
// (cascade prefix pass: 24-ai.news TokenSpeed article, optimisation list,
// hybrid prefix caching) and, at head_dim 128 or 256, 16..64 rows (the
// verify of a speculative draft: zubnet.ai TokenSpeed article, second
// paragraph), and the same with the layer's prologue inline (the fused
// layer entry point at 16..128 rows).  The body and its gfx950 mapping are
// in attn_mfma128_body.h.
#include "attn_mfma128_body.h"

namespace had {
namespace {

// one workgroup per CU (the LDS stage buffers take most of it)
template <int D, int DH>
__global__ __launch_bounds__(64 * kM128Waves, 1) void attn_mfma128_kernel(ValuArgs a) {
  mfma128_partial<D, DH>(a, blockIdx.x, blockIdx.y, blockIdx.z);
}

// the same with the layer's prologue inline
template <int D, int DH>
__global__ __launch_bounds__(64 * kM128Waves, 1) void attn_mfma128_fused_kernel(ValuArgs a, FusedArgs f) {
  mfma128_partial<D, DH, M128FusedStore<D>, true>(a, blockIdx.x, blockIdx.y, blockIdx.z, f);
}

}  // namespace

hipError_t launch_attn_mfma128_fused(const ValuArgs& a_in, const FusedArgs& f, int head_dim, dim3 grid,
                                     hipStream_t stream) {
  // one launch for all rows (16..64 at head_dim >= 128 with wave pairs,
  // 65..128 with a wave per 16 rows), pages of a multiple of 32 tokens, at
  // most kM128New new tokens, rotation partners k-steps apart in one lane
  const int dh = a_in.rows > 64 ? 1 : 2;
  if (a_in.page_size % 32 != 0 || a_in.rows < 16 || a_in.rows > 128 || (dh == 2 && head_dim < 128) ||
      a_in.q_len < 1 || a_in.q_len > kM128New || a_in.num_splits < 1 ||
      !(f.R == 0 || f.R == 64 || (f.R % 128 == 0 && f.R <= head_dim)))
    return hipErrorInvalidValue;
  ValuArgs b = a_in;
  // split ranges of 32-token stages, balanced to within one (a range can
  // start inside a page: one page more than its share)
  const int64_t n_st = static_cast<int64_t>(b.n_pages_plan) * (b.page_size / 32);
  const int64_t st_max = (n_st + b.num_splits - 1) / b.num_splits;
  if ((st_max * 32 + b.page_size - 1) / b.page_size + (b.num_splits > 1 ? 1 : 0) > kMaxPagesPerSplit)
    return hipErrorInvalidValue;
  b.split_base = static_cast<int>(n_st / b.num_splits);
  b.split_rem = static_cast<int>(n_st % b.num_splits);
  b.row_base = 0;
  const dim3 blk(64 * kM128Waves);
  switch (head_dim * 2 + dh - 1) {
    case 128: hipLaunchKernelGGL((attn_mfma128_fused_kernel<64, 1>), grid, blk, 0, stream, b, f); break;
    case 256: hipLaunchKernelGGL((attn_mfma128_fused_kernel<128, 1>), grid, blk, 0, stream, b, f); break;
    case 257: hipLaunchKernelGGL((attn_mfma128_fused_kernel<128, 2>), grid, blk, 0, stream, b, f); break;
    case 512: hipLaunchKernelGGL((attn_mfma128_fused_kernel<256, 1>), grid, blk, 0, stream, b, f); break;
    case 513: hipLaunchKernelGGL((attn_mfma128_fused_kernel<256, 2>), grid, blk, 0, stream, b, f); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

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
