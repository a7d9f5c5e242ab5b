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
// The prefix side is the MFMA partial that stages K and V straight into LDS
// (attn_mfma128_body.h: 16 rows per wave above 64 rows, wave pairs on 16
// rows up to 64 at head_dim >= 128; the register-staged attn_mfma_body.h up
// to 64 rows at head_dim 64), the suffix side the VALU partial in its
// shared-out mode; LDS is the union of the two.
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

// LDS: the two sides' layouts overlaid.  DH: the prefix side's wave
// arrangement in attn_mfma128_body.h (1 or 2), 0 for attn_mfma_body.h.
template <int D, int DH>
union CascadeStore {
  typename std::conditional<DH != 0, M128Lds<D>, MLds<D>>::type m;
  Lds v;
};

template <int D, int DH>
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
    if constexpr (DH != 0) {  // 32-token stages balanced to within one
      const int n_st = px.pages * (P / 32);
      a.split_base = n_st / gp;
      a.split_rem = n_st % gp;
      mfma128_partial<D, DH, CascadeStore<D, DH>>(a, blockIdx.x, blockIdx.y, 0);
    } else {  // whole pages balanced to within one
      a.split_base = px.pages / gp;
      a.split_rem = px.pages % gp;
      mfma_partial<D, false, true, CascadeStore<D, DH>>(a, blockIdx.x, blockIdx.y, 0);
    }
  } else {
    ValuArgs a = as;  // suffix unit blockIdx.x - gp of G - gp, after the prefix's slots
    a.split_offset = gp;
    a.bal_units = G - gp;
    const FusedArgs f{};
    valu_partial<D, false, CascadeStore<D, DH>>(a, f, static_cast<int>(blockIdx.x) - gp, blockIdx.y, 0);
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
  // wave pairs on 16 rows need two groups of four 16-dim output blocks per wave
  const int dh = ap.rows > kMRows ? 1 : (head_dim >= 128 ? 2 : 0);
  switch (head_dim * 4 + dh) {
    case 256: hipLaunchKernelGGL((attn_cascade_kernel<64, 0>), grid, blk, 0, stream, as, px); break;
    case 257: hipLaunchKernelGGL((attn_cascade_kernel<64, 1>), grid, blk, 0, stream, as, px); break;
    case 513: hipLaunchKernelGGL((attn_cascade_kernel<128, 1>), grid, blk, 0, stream, as, px); break;
    case 514: hipLaunchKernelGGL((attn_cascade_kernel<128, 2>), grid, blk, 0, stream, as, px); break;
    case 1025: hipLaunchKernelGGL((attn_cascade_kernel<256, 1>), grid, blk, 0, stream, as, px); break;
    case 1026: hipLaunchKernelGGL((attn_cascade_kernel<256, 2>), grid, blk, 0, stream, as, px); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace had
