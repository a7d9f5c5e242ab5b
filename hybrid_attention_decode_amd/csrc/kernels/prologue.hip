// Fused prologue of a full-attention layer: QK-RMSNorm + partial rotary
// embedding + gate split, with the new K/V rows written straight into their
// KV page slots.  The engine fuses these five steps into one kernel whose
// intermediates never leave registers (zubnet.ai TokenSpeed article, second
// paragraph); here one wave owns one head of one token (the per-row
// arithmetic is in prologue_math.h, shared with the attention kernels that
// run the prologue inline).  Grid: (token, group of 4 heads), 4 waves per
// block; positions pos = seq_lens[s] - T + j.  Gate and v are copied bit for
// bit.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>

#include "../host/status.h"
#include "had.h"
#include "kcommon.h"
#include "prologue_math.h"

using had::fail;

namespace had {
namespace {

constexpr int kWaves = 4;

struct PrologueArgs {
  const uint16_t* qg;
  const uint16_t* k;
  const uint16_t* v;
  const float* w_q;
  const float* w_k;
  const int32_t* page_table;
  const int32_t* seq_lens;
  uint16_t* k_pool;
  uint16_t* v_pool;
  uint16_t* q_out;
  uint16_t* gate_out;
  int32_t* d_err;
  int T, H_q, H_kv, R, num_pages, P, max_pages;
  int max_len;  // a longer sequence is skipped (HAD_DERR_SEQLEN): no K/V row written
  double coef;  // rope_coef(base, R)
  float eps;
};

template <int D>
__global__ __launch_bounds__(256) void prologue_kernel(PrologueArgs a) {
  constexpr int E = D / 64;  // elements per lane: lane l holds d = l + 64 m
  __shared__ float row[kWaves][D];
  const int s = blockIdx.x / a.T, j = blockIdx.x % a.T;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const size_t tok = static_cast<size_t>(s) * a.T + j;
  const int hh = blockIdx.y * kWaves + wave;  // one head per wave
  if (hh >= a.H_q + a.H_kv) return;           // (wave 0 of block row 0 always has a head)
  const bool is_q = hh < a.H_q;
  const int h = is_q ? hh : hh - a.H_q;

  // Every load is issued before the first is used, none under a branch (a
  // load under a branch waits for itself before the branch ends): the row,
  // the row that is only copied (a q head's gate half, a KV head's v row),
  // then the length and the page id that depends on it.
  const uint16_t* src = is_q ? a.qg + (tok * a.H_q + h) * 2 * D : a.k + (tok * a.H_kv + h) * D;
  const uint16_t* side = is_q ? src + D : a.v + (tok * a.H_kv + h) * D;
  RowIn<D> in;
  row_load<D>(in, src, is_q ? a.w_q : a.w_k, lane);
  uint16_t cp[E];
#pragma unroll
  for (int m = 0; m < E; ++m) cp[m] = side[lane + 64 * m];
  const int L = a.seq_lens[s];
  const int pos = L - a.T + j;
  const bool pos_ok = L >= a.T && L <= a.max_len && pos < a.max_pages * a.P;
  const int pid = a.page_table[static_cast<size_t>(s) * a.max_pages + (pos_ok ? pos / a.P : 0)];
  const bool page_ok = pos_ok && pid >= 0 && pid < a.num_pages;
  if (threadIdx.x == 0 && blockIdx.y == 0) {
    if (!pos_ok) set_err(a.d_err, HAD_DERR_SEQLEN);
    else if (!page_ok) set_err(a.d_err, HAD_DERR_PAGE);
  }

  uint16_t y[E];
  row_norm_rope<D>(in, pos, a.R, a.coef, a.eps, row[wave], lane, y);
  if (is_q) {
    uint16_t* qo = a.q_out + (tok * a.H_q + h) * D;
    uint16_t* go = a.gate_out + (tok * a.H_q + h) * D;
#pragma unroll
    for (int m = 0; m < E; ++m) {
      qo[lane + 64 * m] = y[m];
      go[lane + 64 * m] = cp[m];
    }
  } else if (page_ok) {
    const size_t dst = ((static_cast<size_t>(pid) * a.H_kv + h) * a.P + pos % a.P) * D;
#pragma unroll
    for (int m = 0; m < E; ++m) {
      a.k_pool[dst + lane + 64 * m] = y[m];
      a.v_pool[dst + lane + 64 * m] = cp[m];
    }
  }
}

}  // namespace
}  // namespace had

namespace had {

// The prologue of sequences of at most max_len tokens (the attention layer
// passes the length its split plan covers, so a longer sequence, which the
// attention skips, gets no K/V row either).
int launch_qk_norm_rope_gate(const had_qknrg_desc* d, const had_qknrg_ptrs* p, int64_t max_len, void* stream) {
  if (!d || !p) return fail(HAD_ERR_INVALID_ARG, "qk_norm_rope_gate: NULL argument");
  if (d->n_seqs < 0 || d->T < 0 || d->H_q < 1 || d->H_kv < 1)
    return fail(HAD_ERR_INVALID_ARG, "qk_norm_rope_gate: bad sizes (n_seqs=%d T=%d H_q=%d H_kv=%d)", d->n_seqs, d->T,
                d->H_q, d->H_kv);
  if (d->head_dim != 64 && d->head_dim != 128 && d->head_dim != 256)
    return fail(HAD_ERR_UNSUPPORTED_SHAPE, "qk_norm_rope_gate: head_dim %d not in {64,128,256}", d->head_dim);
  if (d->rotary_dim < 0 || d->rotary_dim > d->head_dim || d->rotary_dim % 2 != 0)
    return fail(HAD_ERR_INVALID_ARG, "qk_norm_rope_gate: rotary_dim %d must be even and <= head_dim", d->rotary_dim);
  if (!(d->rope_base > 0.0) || !(d->eps >= 0.f))
    return fail(HAD_ERR_INVALID_ARG, "qk_norm_rope_gate: rope_base must be > 0 and eps >= 0");
  if (d->num_pages < 1 || d->page_size < 1 || d->max_pages < 1)
    return fail(HAD_ERR_INVALID_ARG, "qk_norm_rope_gate: bad page geometry");
  if (!p->qg || !p->k || !p->v || !p->w_q || !p->w_k || !p->page_table || !p->seq_lens || !p->k_pool ||
      !p->v_pool || !p->q_out || !p->gate_out)
    return fail(HAD_ERR_INVALID_ARG, "qk_norm_rope_gate: NULL pointer in ptrs");
  if (d->n_seqs == 0 || d->T == 0) return had::ok();
  had::PrologueArgs a{};
  a.qg = static_cast<const uint16_t*>(p->qg);
  a.k = static_cast<const uint16_t*>(p->k);
  a.v = static_cast<const uint16_t*>(p->v);
  a.w_q = p->w_q;
  a.w_k = p->w_k;
  a.page_table = p->page_table;
  a.seq_lens = p->seq_lens;
  a.k_pool = static_cast<uint16_t*>(p->k_pool);
  a.v_pool = static_cast<uint16_t*>(p->v_pool);
  a.q_out = static_cast<uint16_t*>(p->q_out);
  a.gate_out = static_cast<uint16_t*>(p->gate_out);
  a.d_err = p->d_err;
  a.T = d->T;
  a.H_q = d->H_q;
  a.H_kv = d->H_kv;
  a.R = d->rotary_dim;
  a.num_pages = d->num_pages;
  a.P = d->page_size;
  a.max_pages = d->max_pages;
  a.max_len = static_cast<int>(std::min<int64_t>(max_len, static_cast<int64_t>(d->max_pages) * d->page_size));
  a.coef = had::rope_coef(d->rope_base, d->rotary_dim);
  a.eps = d->eps;
  const dim3 grid(d->n_seqs * d->T, (d->H_q + d->H_kv + 3) / 4), block(256);
  hipStream_t s = static_cast<hipStream_t>(stream);
  switch (d->head_dim) {
    case 64: hipLaunchKernelGGL(had::prologue_kernel<64>, grid, block, 0, s, a); break;
    case 128: hipLaunchKernelGGL(had::prologue_kernel<128>, grid, block, 0, s, a); break;
    default: hipLaunchKernelGGL(had::prologue_kernel<256>, grid, block, 0, s, a); break;
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(HAD_ERR_HIP, "qk_norm_rope_gate: launch: %s", hipGetErrorString(e));
  return had::ok();
}

}  // namespace had

extern "C" int had_qk_norm_rope_gate(const had_qknrg_desc* d, const had_qknrg_ptrs* p, void* stream) {
  if (!d) return fail(HAD_ERR_INVALID_ARG, "qk_norm_rope_gate: NULL argument");
  return had::launch_qk_norm_rope_gate(d, p, static_cast<int64_t>(d->max_pages) * d->page_size, stream);
}
