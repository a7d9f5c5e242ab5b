// Split-K merge of the decode-attention partials.
//
// For query row r of (sequence s, KV head h) with partials (o_i, m_i, l_i)
// from the splits i (m in base-2 units, o and l unnormalised):
//   M = max_i m_i,  w_i = 2^(m_i - M),  out = sum_i w_i o_i / sum_i w_i l_i,
// rounded to bf16 (nearest even).  Splits with m = -inf carry weight 0; a
// row with no visible key at all (sum of weights 0) is written as zeros.
// This is the log-sum-exp merge that makes the split over the context exact
// up to rounding (the split-K step of the decode path; long contexts up to
// 1M tokens, 24-ai.news long-context table).
//
// One 64-lane wave per (row, 64-wide slice of head_dim): lanes read the
// split maxima 64 at a time, then stream the partials with one coalesced
// 256-byte row per split.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "attn_internal.h"
#include "kcommon.h"

namespace had {
namespace {

__global__ __launch_bounds__(64) void attn_combine_kernel(CombineArgs a, int D) {
  __shared__ float wsh[64];
  const int lane = threadIdx.x;
  const int dblk = blockIdx.x;        // 64-wide slice of head_dim
  const int row = blockIdx.y;         // j * G + g
  const int sh_ = blockIdx.z;         // s * H_kv + h
  const int s = sh_ / a.H_kv, h = sh_ % a.H_kv;
  const int ns = a.num_splits;
  const size_t unit0 = static_cast<size_t>(sh_) * ns;
  const float* ml = a.ws_ml;
  const int d = dblk * 64 + lane;

  // pass 1: row maximum over the splits
  float M = -INFINITY;
  for (int i = lane; i < ns; i += 64) M = fmaxf(M, ml[((unit0 + i) * a.rows + row) * 2]);
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) M = fmaxf(M, shfl_xor_f(M, off));
  const float Ms = (M == -INFINITY) ? 0.f : M;

  // pass 2: weighted sums, 64 splits at a time (weights via LDS broadcast)
  float acc = 0.f, lsum = 0.f;
  for (int i0 = 0; i0 < ns; i0 += 64) {
    const int i = i0 + lane;
    float w = 0.f;
    if (i < ns) {
      const float mi = ml[((unit0 + i) * a.rows + row) * 2];
      w = (mi == -INFINITY) ? 0.f : exp2f(mi - Ms);
      lsum += w * ml[((unit0 + i) * a.rows + row) * 2 + 1];
    }
    __syncthreads();
    wsh[lane] = w;
    __syncthreads();
    const int n = min(64, ns - i0);
    if (d < D) {
      const float* op = a.ws_o + ((unit0 + i0) * a.rows + row) * D + d;
      const size_t stride = static_cast<size_t>(a.rows) * D;
      int k = 0;
      for (; k + 4 <= n; k += 4) {
        const float o0 = op[(k + 0) * stride], o1 = op[(k + 1) * stride];
        const float o2 = op[(k + 2) * stride], o3 = op[(k + 3) * stride];
        acc += wsh[k] * o0;
        acc += wsh[k + 1] * o1;
        acc += wsh[k + 2] * o2;
        acc += wsh[k + 3] * o3;
      }
      for (; k < n; ++k) acc += wsh[k] * op[k * stride];
    }
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) lsum += shfl_xor_f(lsum, off);

  if (d < D) {
    const int jq = row / a.G, g = row % a.G;
    const float y = (lsum > 0.f) ? acc / lsum : 0.f;
    a.out[((static_cast<size_t>(s) * a.q_len + jq) * a.H_q + h * a.G + g) * D + d] = f32_to_bf16(y);
  }
}

}  // namespace

hipError_t launch_attn_combine(const CombineArgs& a, int head_dim, hipStream_t stream) {
  dim3 grid((head_dim + 63) / 64, a.rows, a.n_seqs * a.H_kv);
  hipLaunchKernelGGL(attn_combine_kernel, grid, dim3(64), 0, stream, a, head_dim);
  return hipGetLastError();
}

}  // namespace had
