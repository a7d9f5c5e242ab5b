// Split-K GQA decode attention, MFMA path (16 or more query rows per KV
// head, e.g. GQA group 16 x 4 draft tokens when a speculative draft is
// verified: zubnet.ai TokenSpeed article, second paragraph, speculative
// decoding; 24-ai.news long-context table for the context range).
//
// Same operation and partial format as the VALU path: for the rows of one
// (sequence, KV head), softmax(sm_scale q K^T) V over the split's tokens,
// causal inside the draft, written as unnormalised (o, m, l) in base 2.
//
// gfx950 mapping.  One workgroup of 8 waves per split, two teams of 4 waves;
// each iteration stages 64 tokens of K and V in LDS and team t works on
// tokens 32t .. 32t+31 of them, wave w of a team owning query rows
// 16(w mod 4) .. +15 of the launch.  The teams keep separate softmax states
// and are merged through LDS once at the end, so a split writes one partial
// however many tokens it covers.
//  * Staging: global -> registers -> LDS with two register stages in flight
//    (tiles i+1 and i+2 load while tile i is computed) and two LDS buffers,
//    one barrier per iteration.  A thread moves one 16-byte chunk column of
//    TPT consecutive tokens, so its TPT V chunks transpose in registers
//    (v_perm) into TPT-wide runs of each d-row and go to LDS as 8-byte
//    writes; K keeps its row-major layout with 16-byte chunks XOR-swizzled
//    by token row.
//  * S^T = K Q^T with v_mfma_f32_16x16x32_bf16 (A = K rows from LDS, B = q
//    rows held in registers): the C layout leaves each lane 8 token scores
//    of ONE query row, which is exactly the B operand P^T of O^T = V^T P^T
//    once the 32 tokens are taken in the order tau(g, i) = 4g + i (i < 4),
//    16 + 4g + i-4 (i >= 4) -- so P never goes through LDS, and the
//    online-softmax rescale of a lane's O^T accumulators uses the lane's own
//    row state (skipped when no row maximum of the wave moved).
//  * Row maxima and sums combine the 4 lanes of a row with two bpermutes.
// Above 64 rows the 128-row launches go to attn_mfma128.hip when pages hold
// a multiple of 32 tokens (K and V staged straight into LDS); the R128 form
// here (each wave its 16 rows over both halves of every tile, no team
// merge) serves the other page sizes.
#include "attn_mfma_body.h"

namespace had {
namespace {

template <int D, bool R128, bool PAGE32>
__global__ __launch_bounds__(512, 2) void attn_mfma_kernel(ValuArgs a) {
  mfma_partial<D, R128, PAGE32>(a, blockIdx.x, blockIdx.y, blockIdx.z);
}

}  // namespace

hipError_t launch_attn_mfma(const ValuArgs& a_in, int head_dim, dim3 grid, hipStream_t stream) {
  ValuArgs a = a_in;
  // page-granular split ranges (the VALU plan's base and remainder count
  // tiles); one thread per page id of a split
  static_assert(kMWaves * 64 >= kMaxPagesPerSplit, "a split's page ids are read one per thread");
  if (a.num_splits < 1 || (a.n_pages_plan + a.num_splits - 1) / a.num_splits > kMaxPagesPerSplit)
    return hipErrorInvalidValue;
  a.split_base = a.n_pages_plan / a.num_splits;
  a.split_rem = a.n_pages_plan % a.num_splits;
  hipError_t e = hipSuccess;
  // up to 64 rows: the token-split teams; more: 128 rows per launch
  const bool r128 = a.rows > kMRows;
  for (int rb = 0; rb < a.rows && e == hipSuccess; rb += r128 ? 2 * kMRows : kMRows) {
    a.row_base = rb;
    const dim3 blk(64 * kMWaves);
    const bool p32 = a.page_size % 32 == 0;
    if (p32 && (r128 || head_dim >= 128)) {  // K and V staged straight into LDS, 32-token-stage split ranges
      ValuArgs b = a;
      const int64_t n_st = static_cast<int64_t>(a.n_pages_plan) * (a.page_size / 32);
      const int64_t st_max = (n_st + a.num_splits - 1) / a.num_splits;
      // (with several splits a range of stages can start inside a page: one
      // page more than its share)
      if ((st_max * 32 + a.page_size - 1) / a.page_size + (a.num_splits > 1 ? 1 : 0) > kMaxPagesPerSplit)
        return hipErrorInvalidValue;
      b.split_base = static_cast<int>(n_st / a.num_splits);
      b.split_rem = static_cast<int>(n_st % a.num_splits);
      e = launch_attn_mfma128(b, head_dim, r128 ? 1 : 2, grid, stream);
      continue;
    }
    switch (head_dim * 4 + (r128 ? 2 : 0) + (p32 ? 1 : 0)) {
      case 256: hipLaunchKernelGGL((attn_mfma_kernel<64, false, false>), grid, blk, 0, stream, a); break;
      case 257: hipLaunchKernelGGL((attn_mfma_kernel<64, false, true>), grid, blk, 0, stream, a); break;
      case 258: hipLaunchKernelGGL((attn_mfma_kernel<64, true, false>), grid, blk, 0, stream, a); break;
      case 512: hipLaunchKernelGGL((attn_mfma_kernel<128, false, false>), grid, blk, 0, stream, a); break;
      case 513: hipLaunchKernelGGL((attn_mfma_kernel<128, false, true>), grid, blk, 0, stream, a); break;
      case 514: hipLaunchKernelGGL((attn_mfma_kernel<128, true, false>), grid, blk, 0, stream, a); break;
      case 1024: hipLaunchKernelGGL((attn_mfma_kernel<256, false, false>), grid, blk, 0, stream, a); break;
      case 1025: hipLaunchKernelGGL((attn_mfma_kernel<256, false, true>), grid, blk, 0, stream, a); break;
      case 1026: hipLaunchKernelGGL((attn_mfma_kernel<256, true, false>), grid, blk, 0, stream, a); break;
      default: return hipErrorInvalidValue;
    }
    e = hipGetLastError();
  }
  return e;
}

}  // namespace had
