// One-launch cascade decode attention: the prefix pass and the suffix pass of
// a batch that forked one cached prefix (24-ai.news TokenSpeed article,
// hybrid prefix caching; zubnet.ai TokenSpeed article, first paragraph: most
// of an agentic turn's KV is such a shared prefix) run as one grid.
//
// Run one after the other, the two passes each leave HBM idle at their start
// and end, and the prefix pass -- 128 query rows over a 50,000-token prefix
// -- fills only the CUs its page count allows.  Here workgroup g of the G in
// the grid (per KV head) takes part in the prefix pass when g < G_p and is
// suffix unit g - G_p otherwise; G_p is G in proportion to the prefix's share
// of the batch's tiles, computed on the device from the sequence lengths
// (cascade_prefix_units), so a captured graph replays with new lengths.  The
// partials land in one row of G slots per (sequence, KV head): the prefix's
// G_p first, then each sequence's own suffix units, and the usual merge reads
// prefix + own (the merge recomputes the same integers).
//
// The prefix side is the MFMA partial (above 64 rows the one that stages K
// and V straight into LDS, attn_mfma128_body.h), the suffix side the VALU
// partial in its shared-out mode; LDS is the union of the two.
#include "attn_mfma128_body.h"
#include "attn_valu_body.h"

namespace had {
namespace {

// What the prefix side changes in the suffix side's arguments.
struct PrefixSide {
  const int32_t* page_table;  // the prefix's page list
  int rows;                   // every sequence's rows
  int pages;                  // prefix pages (page-table row length, plan)
  int prefix_tiles, weight16, min_pu;  // for cascade_prefix_units
};

// LDS: the two sides' layouts overlaid
template <int D, bool R128>
union CascadeStore {
  typename std::conditional<R128, M128Lds<D>, MLds<D>>::type m;
  Lds v;
};

template <int D, bool R128>
__global__ __launch_bounds__(512, 2) void attn_cascade_kernel(ValuArgs as, PrefixSide px) {
  const int lane = threadIdx.x & 63;
  const int P = as.page_size;
  const int G = static_cast<int>(gridDim.x);
  const int gp = __builtin_amdgcn_readfirstlane(cascade_prefix_units(
      as.seq_lens, as.n_seqs, as.pg_begin * P, as.n_pages_plan * (P / 8), G, px.prefix_tiles, px.weight16, px.min_pu, lane));
  if (static_cast<int>(blockIdx.x) < gp) {
    // prefix split blockIdx.x of gp, whole pages balanced to within one; the
    // rows of every sequence, each seeing the whole prefix
    ValuArgs a = as;
    a.page_table = px.page_table;
    a.n_seqs = 1;
    a.rows = px.rows;
    a.max_pages = px.pages;
    a.n_pages_plan = px.pages;
    a.pg_begin = 0;
    a.split_offset = 0;
    a.batch_rows = as.rows;
    a.fixed_len = px.pages * P;
    a.bal_units = 0;
    if constexpr (R128) {  // 32-token stages balanced to within one
      const int n_st = px.pages * (P / 32);
      a.split_base = n_st / gp;
      a.split_rem = n_st % gp;
      mfma128_partial<D, 1, CascadeStore<D, R128>>(a, blockIdx.x, blockIdx.y, 0);
    } else {  // whole pages balanced to within one
      a.split_base = px.pages / gp;
      a.split_rem = px.pages % gp;
      mfma_partial<D, false, true, CascadeStore<D, R128>>(a, blockIdx.x, blockIdx.y, 0);
    }
  } else {
    ValuArgs a = as;  // suffix unit blockIdx.x - gp of G - gp, after the prefix's slots
    a.split_offset = gp;
    a.bal_units = G - gp;
    const FusedArgs f{};
    valu_partial<D, false, CascadeStore<D, R128>>(a, f, static_cast<int>(blockIdx.x) - gp, blockIdx.y, 0);
  }
}

}  // namespace

hipError_t launch_attn_cascade(const ValuArgs& ap, const ValuArgs& as, int prefix_tiles, int weight16, int min_pu,
                               int head_dim, dim3 grid, hipStream_t stream) {
  // one launch covers at most 128 prefix rows and 8 rows per sequence, pages
  // of a multiple of 32 tokens (the host checks; these keep a bad call out)
  if (ap.rows < 1 || ap.rows > 2 * kMRows || as.rows > kRows || ap.page_size % 32 != 0 || as.bal_units != 0 ||
      ap.n_pages_plan != ap.max_pages || ap.batch_rows != as.rows || static_cast<int>(grid.x) < min_pu + as.n_seqs ||
      min_pu < 1 || (ap.n_pages_plan + min_pu - 1) / min_pu + 1 > kMaxPagesPerSplit || weight16 < 1 || weight16 > 256)
    return hipErrorInvalidValue;
  const PrefixSide px{ap.page_table, ap.rows, ap.n_pages_plan, prefix_tiles, weight16, min_pu};
  const dim3 blk(64 * kMWaves);
  const bool r128 = ap.rows > kMRows;
  switch (head_dim * 2 + (r128 ? 1 : 0)) {
    case 128: hipLaunchKernelGGL((attn_cascade_kernel<64, false>), grid, blk, 0, stream, as, px); break;
    case 129: hipLaunchKernelGGL((attn_cascade_kernel<64, true>), grid, blk, 0, stream, as, px); break;
    case 256: hipLaunchKernelGGL((attn_cascade_kernel<128, false>), grid, blk, 0, stream, as, px); break;
    case 257: hipLaunchKernelGGL((attn_cascade_kernel<128, true>), grid, blk, 0, stream, as, px); break;
    case 512: hipLaunchKernelGGL((attn_cascade_kernel<256, false>), grid, blk, 0, stream, as, px); break;
    case 513: hipLaunchKernelGGL((attn_cascade_kernel<256, true>), grid, blk, 0, stream, as, px); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace had
