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

// Work units of a batch's suffix pass shared out by length: sequence t has
// n_t tiles of 8 tokens from token tok_begin on; every sequence with a tile
// gets one unit and the units left over are given in proportion to n_t
// (floor), so sum W_t <= G.  Lane t of the calling wave returns sequence t's
// n_t, W_t and first unit O_t (n_seqs <= 64); every wave that calls it with
// the same lengths gets the same integers, so the partial kernel and the
// merge agree without exchanging anything.
__device__ __forceinline__ void bal_share(const int32_t* seq_lens, int n_seqs, int tok_begin, int max_tiles, int G,
                                          int lane, int& n_t, int& W_t, int& O_t) {
  const int L = lane < n_seqs ? seq_lens[lane] : 0;
  n_t = lane < n_seqs ? min(max(0, (L - tok_begin + 7) / 8), max_tiles) : 0;
  const int K = __popcll(__ballot(n_t > 0));
  long long N = n_t;
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) N += __shfl_xor(N, off);
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

// Inputs of the prologue when the VALU attention kernel runs it inline (the
// fused layer entry point, below 16 query rows per KV head): every
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
  // its num_splits slots (W_s from bal_share over seq_lens)
  const int32_t* seq_lens;
  int bal_units, prefix_splits, tok_begin, max_tiles;
};

hipError_t launch_attn_valu(const ValuArgs& a, int head_dim, dim3 grid, hipStream_t stream);
hipError_t launch_attn_valu_fused(const ValuArgs& a, const FusedArgs& f, int head_dim, dim3 grid, hipStream_t stream);
hipError_t launch_attn_mfma(const ValuArgs& a, int head_dim, dim3 grid, hipStream_t stream);
hipError_t launch_attn_combine(const CombineArgs& a, int head_dim, hipStream_t stream);

}  // namespace had
