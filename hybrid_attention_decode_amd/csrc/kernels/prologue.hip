// Fused prologue of a full-attention layer: QK-RMSNorm + partial rotary
// embedding + gate split, with the new K/V rows written straight into their
// KV page slots.  The engine fuses these five steps into one kernel whose
// intermediates never leave registers (zubnet.ai TokenSpeed article, second
// paragraph); here one wave owns one head of one token and the only other
// storage touched is a 1 KB LDS row used to fetch the rotation partner.
// Grid: (token, group of 4 heads), 4 waves per block.
//
//   q    = RMSNorm(qg[.., 0, :]) * w_q,   gate = qg[.., 1, :]
//   k    = RMSNorm(k) * w_k,              v unchanged
//   RMSNorm(x) = x / sqrt(mean(x^2) + eps)                       (fp32)
//   dims d < R rotate in pairs (i, i + R/2), angle pos * base^(-2i/R):
//     y_i' = y_i cos - y_{i+R/2} sin,  y_{i+R/2}' = y_{i+R/2} cos + y_i sin
//   (RMSNorm: Zhang & Sennrich 2019; rotary embedding: Su et al., RoFormer
//   2021, applied to a prefix of the head), angles in fp64 (reduced to
//   [-pi, pi] before an fp32 sine/cosine), pos = seq_lens[s] - T + j.
// Outputs are rounded to bf16 (nearest even); gate and v are copied bit for
// bit.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../host/status.h"
#include "had.h"
#include "kcommon.h"

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
  double base;
  float eps;
};

template <int D>
__global__ __launch_bounds__(256) void prologue_kernel(PrologueArgs a) {
  constexpr int E = D / 64;  // elements per lane: lane l holds d = l + 64 m
  __shared__ float row[kWaves][D];
  const int s = blockIdx.x / a.T, j = blockIdx.x % a.T;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int L = a.seq_lens[s];
  const int pos = L - a.T + j;
  const bool pos_ok = L >= a.T && pos < a.max_pages * a.P;
  int pid = -1;
  if (pos_ok) pid = a.page_table[static_cast<size_t>(s) * a.max_pages + pos / a.P];
  const bool page_ok = pos_ok && pid >= 0 && pid < a.num_pages;
  if (threadIdx.x == 0 && blockIdx.y == 0) {
    if (!pos_ok) set_err(a.d_err, HAD_DERR_SEQLEN);
    else if (!page_ok) set_err(a.d_err, HAD_DERR_PAGE);
  }
  const size_t tok = static_cast<size_t>(s) * a.T + j;

  // rotation angle of this lane's pair index (i = d mod R/2 for d < R):
  // theta = pos * base^(-2i/R) in fp64 (at pos ~ 1e6 an fp32 product would
  // be off by ~0.06 rad), reduced to [-pi, pi] in fp64, then sine and cosine
  // of the small reduced angle in fp32.
  const int half = a.R / 2;
  const double log2_base = log2(a.base);
  float cs[E], sn[E];
#pragma unroll
  for (int m = 0; m < E; ++m) {
    const int d = lane + 64 * m;
    cs[m] = 1.f;
    sn[m] = 0.f;
    if (d < a.R) {
      const int i = d % half;
      const double inv_freq = exp2(-2.0 * i / a.R * log2_base);
      const double theta = static_cast<double>(pos) * inv_freq;
      const double two_pi = 6.283185307179586476925286766559;
      const double red = theta - two_pi * rint(theta / two_pi);
      sincosf(static_cast<float>(red), &sn[m], &cs[m]);
    }
  }

  {
    const int hh = blockIdx.y * kWaves + wave;  // one head per wave
    if (hh >= a.H_q + a.H_kv) return;
    const bool is_q = hh < a.H_q;
    const int h = is_q ? hh : hh - a.H_q;
    const uint16_t* src = is_q ? a.qg + (tok * a.H_q + h) * 2 * D : a.k + (tok * a.H_kv + h) * D;
    const float* w = is_q ? a.w_q : a.w_k;
    float x[E];
    float ss = 0.f;
#pragma unroll
    for (int m = 0; m < E; ++m) {
      x[m] = bf16_to_f32(src[lane + 64 * m]);
      ss += x[m] * x[m];
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) ss += shfl_xor_f(ss, off);
    const float inv = 1.f / sqrtf(ss / static_cast<float>(D) + a.eps);
#pragma unroll
    for (int m = 0; m < E; ++m) {
      x[m] = x[m] * inv * w[lane + 64 * m];
      row[wave][lane + 64 * m] = x[m];
    }
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
    uint16_t y[E];
#pragma unroll
    for (int m = 0; m < E; ++m) {
      const int d = lane + 64 * m;
      float r = x[m];
      if (d < a.R) {
        const float other = row[wave][d < half ? d + half : d - half];
        r = d < half ? x[m] * cs[m] - other * sn[m] : x[m] * cs[m] + other * sn[m];
      }
      y[m] = f32_to_bf16(r);
    }
    __builtin_amdgcn_wave_barrier();
    if (is_q) {
      uint16_t* qo = a.q_out + (tok * a.H_q + h) * D;
      uint16_t* go = a.gate_out + (tok * a.H_q + h) * D;
      const uint16_t* gi = src + D;
#pragma unroll
      for (int m = 0; m < E; ++m) {
        qo[lane + 64 * m] = y[m];
        go[lane + 64 * m] = gi[lane + 64 * m];
      }
    } else if (page_ok) {
      const size_t dst = ((static_cast<size_t>(pid) * a.H_kv + h) * a.P + pos % a.P) * D;
      const uint16_t* vi = a.v + (tok * a.H_kv + h) * D;
#pragma unroll
      for (int m = 0; m < E; ++m) {
        a.k_pool[dst + lane + 64 * m] = y[m];
        a.v_pool[dst + lane + 64 * m] = vi[lane + 64 * m];
      }
    }
  }
}

}  // namespace
}  // namespace had

extern "C" int had_qk_norm_rope_gate(const had_qknrg_desc* d, const had_qknrg_ptrs* p, void* stream) {
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
  a.base = d->rope_base;
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
