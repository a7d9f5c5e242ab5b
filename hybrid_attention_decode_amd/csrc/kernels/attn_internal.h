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
  int n_pages_plan;  // pages the split plan covers (n).  VALU kernel: split i owns the 8-token tiles
                     // [i*N/ns, (i+1)*N/ns) of the N = n*page_size/8 tiles (its first and last page
                     // possibly shared with a neighbour); MFMA kernel: the pages [i*n/ns, (i+1)*n/ns)
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
};

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
};

hipError_t launch_attn_valu(const ValuArgs& a, int head_dim, dim3 grid, hipStream_t stream);
hipError_t launch_attn_valu_fused(const ValuArgs& a, const FusedArgs& f, int head_dim, dim3 grid, hipStream_t stream);
hipError_t launch_attn_mfma(const ValuArgs& a, int head_dim, dim3 grid, hipStream_t stream);
hipError_t launch_attn_combine(const CombineArgs& a, int head_dim, hipStream_t stream);

}  // namespace had
