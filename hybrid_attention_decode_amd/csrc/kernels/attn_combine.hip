// Split-K merge of the decode-attention partials.
//
// For query row r of (sequence s, KV head h) with partials (o_i, m_i, l_i)
// from the splits i (m in base-2 units, o and l unnormalised):
//   M = max_i m_i,  w_i = 2^(m_i - M),  out = sum_i w_i o_i / sum_i w_i l_i,
// rounded to bf16 (nearest even) -- after an optional multiplication by
// sigmoid(gate) (the gated attention output of the full-attention layers).
// Splits with m = -inf carry weight 0; a row with no visible key at all (sum
// of weights 0) is written as zeros.
// This log-sum-exp merge makes the split over the context exact up to
// rounding (long contexts up to 1M tokens, 24-ai.news long-context table).
//
// The merge reads every partial once (rows x splits x head_dim fp32) and is
// bound by memory latency and by how many CUs pull the partials, not by
// HBM bandwidth: one 4-wave block per (row, 32-dim slice) -- 8 blocks per
// row at head_dim 256 -- issues all of its partial loads (float4 per lane,
// up to 256 splits per pass) before it touches any of them, reads the
// maxima in the same round trip, and reduces across waves through LDS.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "attn_internal.h"
#include "kcommon.h"

namespace had {
namespace {

constexpr int kWaves = 4;
constexpr int kDC = 32;                      // output dims per block
constexpr int kLS = kDC / 4;                 // lanes per split row (float4 each)
constexpr int kSPW = 64 / kLS;               // split rows per wave per load
constexpr int kU = 8;                        // loads per lane per pass
constexpr int kPass = kWaves * kSPW * kU;    // splits per pass (256)
static_assert(kPass <= 64 * kWaves, "one maximum per thread per pass");

__global__ __launch_bounds__(64 * kWaves) void attn_combine_kernel(CombineArgs a, int D) {
  __shared__ float wsh[kPass];
  __shared__ float4 red[kWaves][kLS];
  __shared__ float scal[kWaves];
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int sub = lane / kLS, dl = lane % kLS;
  const int row = blockIdx.x;
  const int d0 = blockIdx.y * kDC;
  const int unit = blockIdx.z;  // s * H_kv + h
  const int ns = a.num_splits;
  const size_t base = static_cast<size_t>(unit) * ns;
  const float* ml = a.ws_ml;
  const size_t ostride4 = static_cast<size_t>(a.rows) * D / 4;  // float4s between consecutive splits
  const float4* o4 = reinterpret_cast<const float4*>(a.ws_o + (base * a.rows + row) * D + d0);
  const int s = unit / a.H_kv, h = unit % a.H_kv;
  const int jq = row / a.G, g = row % a.G;
  const size_t head = (static_cast<size_t>(s) * a.q_len + jq) * a.H_q + h * a.G + g;
  // the gate is read in the same round trip as the partials (unconditionally:
  // without a gate the load reads the output row, and the value is unused)
  const uint2 gw = *reinterpret_cast<const uint2*>(
      a.gate ? a.gate + head * a.gate_hstride + d0 + 4 * (tid % kLS) : a.out + head * D + d0 + 4 * (tid % kLS));

  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  float M = -INFINITY;
  float lsum = 0.f;
  for (int p0 = 0; p0 < ns; p0 += kPass) {
    // issue every load of this pass first
    float4 ov[kU];
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      const int i = p0 + (u * kWaves + wave) * kSPW + sub;
      ov[u] = (i < ns) ? o4[i * ostride4 + dl] : make_float4(0.f, 0.f, 0.f, 0.f);
    }
    float mi = -INFINITY, li = 0.f;
    const int my = p0 + tid;  // this thread's split for the maxima
    if (tid < kPass && my < ns) {
      mi = ml[((base + my) * a.rows + row) * 2];
      li = ml[((base + my) * a.rows + row) * 2 + 1];
    }
    // block maximum of this pass, merged into the running maximum
    float mw = mi;
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) mw = fmaxf(mw, shfl_xor_f(mw, off));
    if (lane == 0) scal[wave] = mw;
    __syncthreads();
    float mp = scal[0];
#pragma unroll
    for (int w = 1; w < kWaves; ++w) mp = fmaxf(mp, scal[w]);
    const float M_new = fmaxf(M, mp);
    const float Ms = (M_new == -INFINITY) ? 0.f : M_new;
    const float rescale = (M == -INFINITY) ? 0.f : exp2f(M - Ms);
    acc.x *= rescale; acc.y *= rescale; acc.z *= rescale; acc.w *= rescale;
    lsum *= rescale;
    M = M_new;
    if (tid < kPass && my < ns) {
      const float w = (mi == -INFINITY) ? 0.f : exp2f(mi - Ms);
      wsh[tid] = w;
      lsum += w * li;
    }
    __syncthreads();
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      const int il = (u * kWaves + wave) * kSPW + sub;
      if (p0 + il < ns) {
        const float w = wsh[il];
        acc.x += w * ov[u].x; acc.y += w * ov[u].y; acc.z += w * ov[u].z; acc.w += w * ov[u].w;
      }
    }
    __syncthreads();
  }
  // sum over the split sub-rows of a wave, then over the waves
#pragma unroll
  for (int off = kLS; off < 64; off <<= 1) {
    acc.x += shfl_xor_f(acc.x, off); acc.y += shfl_xor_f(acc.y, off);
    acc.z += shfl_xor_f(acc.z, off); acc.w += shfl_xor_f(acc.w, off);
  }
  if (sub == 0) red[wave][dl] = acc;
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) lsum += shfl_xor_f(lsum, off);
  if (lane == 0) scal[wave] = lsum;
  __syncthreads();
  if (tid < kLS) {
    float4 t = red[0][tid];
    float l = scal[0];
#pragma unroll
    for (int w = 1; w < kWaves; ++w) {
      t.x += red[w][tid].x; t.y += red[w][tid].y; t.z += red[w][tid].z; t.w += red[w][tid].w;
      l += scal[w];
    }
    const float inv = (l > 0.f) ? 1.f / l : 0.f;
    float4 r = make_float4(t.x * inv, t.y * inv, t.z * inv, t.w * inv);
    if (a.gate) {  // gated output: sigmoid(gate) in fp32, before the rounding
      r.x *= 1.f / (1.f + expf(-bf16_lo(gw.x)));
      r.y *= 1.f / (1.f + expf(-bf16_hi(gw.x)));
      r.z *= 1.f / (1.f + expf(-bf16_lo(gw.y)));
      r.w *= 1.f / (1.f + expf(-bf16_hi(gw.y)));
    }
    uint16_t* op = a.out + head * D + d0 + 4 * tid;
    *reinterpret_cast<uint2*>(op) = make_uint2(pack_bf16x2(r.x, r.y), pack_bf16x2(r.z, r.w));
  }
}

}  // namespace

hipError_t launch_attn_combine(const CombineArgs& a, int head_dim, hipStream_t stream) {
  if (head_dim != 64 && head_dim != 128 && head_dim != 256) return hipErrorInvalidValue;
  const dim3 grid(a.rows, head_dim / kDC, a.n_seqs * a.H_kv);
  hipLaunchKernelGGL(attn_combine_kernel, grid, dim3(64 * kWaves), 0, stream, a, head_dim);
  return hipGetLastError();
}

}  // namespace had
