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
  int n_pages_plan;  // pages the split plan covers; split i owns [i*n/ns, (i+1)*n/ns)
  int deterministic;  // fixed tile stride per wave instead of dynamic claims
  float scale_log2;
};

struct CombineArgs {
  const float* ws_o;
  const float* ws_ml;
  uint16_t* out;
  int n_seqs, q_len, H_q, H_kv, G, rows, num_splits;
};

hipError_t launch_attn_valu(const ValuArgs& a, int head_dim, dim3 grid, hipStream_t stream);
hipError_t launch_attn_mfma(const ValuArgs& a, int head_dim, dim3 grid, hipStream_t stream);
hipError_t launch_attn_combine(const CombineArgs& a, int head_dim, hipStream_t stream);

}  // namespace had
