// Internal launch interface between the decode-attention host code and its
// kernels (not part of the C ABI).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "had.h"

namespace had {

// Largest page range one split-K work unit may own (its page ids are staged
// in LDS).
constexpr int kMaxPagesPerSplit = 512;
// Largest number of splits the merge kernel accepts per (sequence, KV head).
constexpr int kMaxSplits = 4096;

struct ValuArgs {
  const uint16_t* q;
  const uint16_t* k_pool;
  const uint16_t* v_pool;
  const int32_t* page_table;
  const int32_t* seq_lens;
  float* ws_o;
  float* ws_ml;
  int32_t* d_err;
  int n_seqs, q_len, H_q, H_kv, G, rows, row_base;
  int num_pages, page_size, max_pages, num_splits, pps;
  int n_pages_plan;  // pages the split plan covers (n).  VALU kernel: of the N = n*page_size/8 tiles of 8
                     // tokens split i owns [i*base + min(i, rem), (i+1)*base + min(i+1, rem)) with
                     // base = N / ns, rem = N % ns (the first rem splits one tile more; a split's first
                     // and last page possibly shared with a neighbour); MFMA kernel: the pages
                     // [i*b + min(i, r), (i+1)*b + min(i+1, r)) with b = n / ns, r = n % ns
  int split_base, split_rem;  // N / ns and N % ns of the VALU plan, n / ns and n % ns of the MFMA
                              // plan (host side)
  int deterministic;  // fixed tile stride per wave instead of dynamic claims
  float scale_log2;
  // Shared-prefix (cascade) passes.  Defaults (0, 0, num_splits, rows, 0, -1)
  // give the plain split-K launch.
  int pg_begin;      // the plan covers page-table entries pg_begin .. pg_begin + n_pages_plan
  int split_offset;  // partial of split sp goes to workspace split split_offset + sp ...
  int ns_total;      // ... of ns_total per (sequence, KV head)
  int ws_rows;       // query rows per (sequence, KV head) in the workspace
  int batch_rows;    // MFMA prefix pass: > 0 = the launch's rows are those of all sequences
                     // (row r belongs to sequence r / batch_rows); page table row 0 is the prefix
  int fixed_len;     // >= 0: every row sees exactly this many tokens (the prefix), seq_lens unused
  int bal_units;     // > 0 (suffix pass of the cascade, VALU): the launch's blockIdx.x is one of bal_units
                     // work units shared out over the sequences in proportion to their suffix length
                     // (bal_share below); 0 = the split plan above
};

// LDS of a kernel, one variable per storage type T: a partial body names its
// part of g_lds<Store> directly (Store = its own layout, or the union of both
// layouts in the one-launch cascade), so every LDS address stays a constant
// offset of one variable -- reached through a reference parameter instead,
// the compiler no longer pairs neighbouring reads into one instruction and
// the 128-row MFMA partial runs out of registers.
namespace {
template <class T>
__shared__ T g_lds;
}  // namespace

// Suffix tiles of a batch: lane t of the calling wave gets sequence t's
// n_t, the tiles of 8 tokens from token tok_begin on (at most max_tiles);
// every lane gets K, the number of sequences with a tile, and N, the total
// (n_seqs <= 64).
__device__ __forceinline__ void suffix_tiles(const int32_t* seq_lens, int n_seqs, int tok_begin, int max_tiles,
                                             int lane, int& n_t, int& K, long long& N) {
  const int L = lane < n_seqs ? seq_lens[lane] : 0;
  n_t = lane < n_seqs ? min(max(0, (L - tok_begin + 7) / 8), max_tiles) : 0;
  K = __popcll(__ballot(n_t > 0));
  N = n_t;
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) N += __shfl_xor(N, off);
}

// Work units of a batch's suffix pass shared out by length: sequence t has
// n_t tiles of 8 tokens from token tok_begin on; every sequence with a tile
// gets one unit and the units left over are given in proportion to n_t
// (floor), so sum W_t <= G.  Lane t of the calling wave returns sequence t's
// n_t, W_t and first unit O_t (n_seqs <= 64); every wave that calls it with
// the same lengths gets the same integers, so the partial kernel and the
// merge agree without exchanging anything.
__device__ __forceinline__ void bal_share(const int32_t* seq_lens, int n_seqs, int tok_begin, int max_tiles, int G,
                                          int lane, int& n_t, int& W_t, int& O_t) {
  int K;
  long long N;
  suffix_tiles(seq_lens, n_seqs, tok_begin, max_tiles, lane, n_t, K, N);
  const long long spare = G > K ? G - K : 0;
  W_t = n_t > 0 ? 1 + static_cast<int>(spare * n_t / (N > 0 ? N : 1)) : 0;
  int x = W_t;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int y = __shfl_up(x, off);
    if (lane >= off) x += y;
  }
  O_t = x - W_t;
}

// One-launch cascade: G workgroups do both passes, the first G_p the prefix
// pass (prefix_tiles tiles of 8 tokens, read once for the rows of every
// sequence) and the rest the suffixes, shared out by bal_share.  G_p is G in
// proportion to the prefix's cost against the suffixes' (rounded), a prefix
// tile costing weight16 / 16 suffix tiles, at least min_pu (so that no prefix
// split exceeds the page cap) and at most G - K (one unit for each sequence
// with a suffix; the host guarantees min_pu + n_seqs <= G).  The same integer
// in every wave that calls it with the same lengths.
__device__ __forceinline__ int cascade_prefix_units(const int32_t* seq_lens, int n_seqs, int tok_begin, int max_tiles,
                                                    int G, int prefix_tiles, int weight16, int min_pu, int lane) {
  int n_t, K;
  long long N;
  suffix_tiles(seq_lens, n_seqs, tok_begin, max_tiles, lane, n_t, K, N);
  const long long T = static_cast<long long>(prefix_tiles) * weight16, tot = T + 16 * N;
  long long gp = (2 * static_cast<long long>(G) * T + tot) / (2 * tot);
  gp = gp < min_pu ? min_pu : gp;
  gp = gp > G - max(K, 1) ? G - max(K, 1) : gp;  // (one suffix unit at least: it reports short sequences)
  return static_cast<int>(gp);
}

// Inputs of the prologue when an attention kernel runs it inline (the fused
// layer entry point: the VALU partial below 16 query rows per KV head, the
// MFMA partial that loads K and V straight into LDS at 16..128): every
// workgroup normalises and rotates its own query rows; the workgroup whose
// split holds the last position also normalises and rotates the new keys,
// writes the new K/V rows to the pools and adds the new tokens to its
// partial from on-chip copies.
struct FusedArgs {
  const uint16_t* qg;     // [n_seqs][q_len][H_q][2][D]: q, then gate
  const uint16_t* k_new;  // [n_seqs][q_len][H_kv][D] before norm / rotation
  const uint16_t* v_new;  // [n_seqs][q_len][H_kv][D]
  const float* w_q;
  const float* w_k;
  uint16_t* k_pool;       // the pools again, writable
  uint16_t* v_pool;
  uint16_t* gate_out;     // [n_seqs][q_len][H_q][D]
  uint16_t* q_out;        // optional, same layout
  double rope_coef;       // -2 log2(rope base) / R (rope_coef())
  float eps;
  int R;                  // rotary dims
};

struct CombineArgs {
  const float* ws_o;
  const float* ws_ml;
  uint16_t* out;
  int n_seqs, q_len, H_q, H_kv, G, rows, num_splits;
  // optional output gate: out *= sigmoid(gate), gate of (s, j, hq) at
  // gate + ((s * q_len + j) * H_q + hq) * gate_hstride (the gate half of qg)
  const uint16_t* gate;
  int gate_hstride;
  // merge of a cascade whose suffix pass shared out bal_units work units
  // (ValuArgs::bal_units): sequence s merges prefix_splits + W_s partials of
  // its num_splits slots (W_s from bal_share over seq_lens).  One-launch
  // cascade (prefix_tiles > 0): bal_units is the launch's G units of both
  // passes, prefix_splits = cascade_prefix_units(...) and the suffixes share
  // the other G - prefix_splits.
  const int32_t* seq_lens;
  int bal_units, prefix_splits, tok_begin, max_tiles;
  int prefix_tiles, prefix_weight16, min_prefix_units;
};

hipError_t launch_attn_valu(const ValuArgs& a, int head_dim, dim3 grid, hipStream_t stream);
hipError_t launch_attn_valu_fused(const ValuArgs& a, const FusedArgs& f, int head_dim, dim3 grid, hipStream_t stream);
hipError_t launch_attn_mfma(const ValuArgs& a, int head_dim, dim3 grid, hipStream_t stream);
// the MFMA partial that loads K and V straight into LDS with the layer's
// prologue inline: 16..128 rows in one launch (16..64 at head_dim >= 128),
// pages of a multiple of 32 tokens, q_len <= 8, rotary dims 0, 64 or a
// multiple of 128; a.split_base / split_rem are recomputed as stage ranges
hipError_t launch_attn_mfma128_fused(const ValuArgs& a, const FusedArgs& f, int head_dim, dim3 grid,
                                     hipStream_t stream);
// both cascade passes in one grid (grid.x = G units per KV head): prefix args
// ap as for the MFMA prefix pass, suffix args as as for the shared-out suffix
// pass with bal_units 0 (set per workgroup), ns_total = G in both
hipError_t launch_attn_cascade(const ValuArgs& ap, const ValuArgs& as, int prefix_tiles, int weight16, int min_pu,
                               int head_dim, dim3 grid, hipStream_t stream);
// cost of a prefix tile in suffix tiles (x16) in the one-launch cascade's
// unit split, measured with both sides running: a 64-token page costs the
// 128-row MFMA side (K and V staged straight into LDS, ranges of 32-token
// stages) about 1.3x what it costs the 8-row VALU side (16 x 50K prefix, one
// launch + merge: the weights 14 / 17 / 20 / 23 / 28 gave 48.0 / 46.6 /
// 44.3-45.8 / 44.7 / 45.7-46.7 us, a smaller weight also leaving fewer
// 128-row partials to merge); up to 64 rows the MFMA side streams at about
// the VALU side's rate
inline int cascade_prefix_weight16(int prefix_rows) { return prefix_rows > 64 ? 21 : 18; }
hipError_t launch_attn_combine(const CombineArgs& a, int head_dim, hipStream_t stream);
// had_qk_norm_rope_gate for sequences of at most max_len tokens (longer ones
// are skipped with HAD_DERR_SEQLEN)
int launch_qk_norm_rope_gate(const had_qknrg_desc* d, const had_qknrg_ptrs* p, int64_t max_len, void* stream);

}  // namespace had
