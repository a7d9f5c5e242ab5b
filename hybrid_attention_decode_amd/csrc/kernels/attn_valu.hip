// Split-K GQA decode attention, VALU path (query rows per KV head < 16).
//
// Operation: softmax(sm_scale * q K^T) V over the paged context of one
// sequence and KV head, for up to 8 query rows at once (GQA group x draft
// tokens), split over the context; each workgroup writes one unnormalised
// partial (o, m, l) that a separate kernel merges.  Full-attention layers of
// the hybrid model (24-ai.news TokenSpeed article, model paragraph), paged KV
// (zubnet.ai TokenSpeed article, second paragraph), contexts to 1M tokens
// (24-ai.news long-context table).
//
// gfx950 mapping (one workgroup = 8 waves, two per SIMD, each wave streams
// its own tiles of 8 tokens; the workgroup owns a contiguous range of
// tiles, balanced to within one tile, one workgroup per CU):
//  * QK: a tile step covers TPS tokens with LPT lanes per token; lane j of a
//    token loads 16-byte chunks j, j+LPT of the K row (coalesced 128-bit
//    loads straight into registers) and accumulates all 8 rows with
//    v_dot2c_f32_bf16 against q held in registers.  q is stored in a
//    lane-dependent row order (slot s of lane j holds row s ^ sigma(j)) so the
//    cross-lane sum is a reduce-scatter of 7 DPP adds after which lane j holds
//    the full score of row sigma(j): no lane idles and no selects are needed.
//  * Online softmax in base 2 (scores prescaled by sm_scale*log2 e), row max
//    by DPP/bpermute across the tile, p rounded once to bf16 and used for
//    both the numerator and the running sum.
//  * PV: lanes own 4 consecutive d of V rows (coalesced 64-bit loads); p
//    pairs of two tokens are broadcast through LDS and v pairs are formed
//    with v_perm_b32, so every MAC is a bf16 dot2.
//  * K/V of a wave's next two tiles are in flight while it computes one;
//    tiles after the first two are claimed from an LDS counter.
//  * The 8 waves' partials are merged through LDS before the single store.
#include "attn_valu_body.h"

namespace had {

namespace {

template <int D, bool FUSED>
__global__ __launch_bounds__(512, 2) void attn_valu_kernel(ValuArgs a, FusedArgs f) {
  valu_partial<D, FUSED>(a, f, blockIdx.x, blockIdx.y, blockIdx.z);
}

}  // namespace

hipError_t launch_attn_valu(const ValuArgs& a, int head_dim, dim3 grid, hipStream_t stream) {
  const FusedArgs f{};
  switch (head_dim) {
    case 64: hipLaunchKernelGGL((attn_valu_kernel<64, false>), grid, dim3(64 * kWaves), 0, stream, a, f); break;
    case 128: hipLaunchKernelGGL((attn_valu_kernel<128, false>), grid, dim3(64 * kWaves), 0, stream, a, f); break;
    case 256: hipLaunchKernelGGL((attn_valu_kernel<256, false>), grid, dim3(64 * kWaves), 0, stream, a, f); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_attn_valu_fused(const ValuArgs& a, const FusedArgs& f, int head_dim, dim3 grid, hipStream_t stream) {
  if (a.q_len > kRows) return hipErrorInvalidValue;  // one new-token key row per wave
  switch (head_dim) {
    case 64: hipLaunchKernelGGL((attn_valu_kernel<64, true>), grid, dim3(64 * kWaves), 0, stream, a, f); break;
    case 128: hipLaunchKernelGGL((attn_valu_kernel<128, true>), grid, dim3(64 * kWaves), 0, stream, a, f); break;
    case 256: hipLaunchKernelGGL((attn_valu_kernel<256, true>), grid, dim3(64 * kWaves), 0, stream, a, f); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace had
