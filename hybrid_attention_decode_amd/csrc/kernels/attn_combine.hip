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
// row at head_dim 256, or 16-dim slices when that leaves under 256 blocks --
// issues all of its partial loads (float4 per lane, up to 256 splits per
// pass) and their maxima before it touches any of them.
// Each wave merges its own 64 splits of a pass in registers against its own
// running maximum (lane swaps across the split rows, no LDS), and the four
// waves' results are merged once through LDS, rescaled to the block's
// maximum: one barrier per block.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "attn_internal.h"
#include "kcommon.h"

namespace had {
namespace {

constexpr int kWaves = 4;
constexpr int kPass = 256;  // splits per pass

// max (sum) over the split rows of a wave, the lanes congruent to l mod LS:
// rotations by 4 and 8 inside each 16-lane row, then lanes l ^ 16 and l ^ 32
template <int LS>
__device__ __forceinline__ float max_rows(float x) {
  if constexpr (LS == 4) x = fmaxf(x, dpp<DPP_ROW_ROR4>(x));
  x = fmaxf(x, dpp<DPP_ROW_ROR8>(x));
  return max_xor32(max_xor16(x));
}
template <int LS>
__device__ __forceinline__ float sum_rows(float x) {
  if constexpr (LS == 4) x += dpp<DPP_ROW_ROR4>(x);
  x += dpp<DPP_ROW_ROR8>(x);
  return sum_xor32(sum_xor16(x));
}

// DC output dims per block: 32, or 16 when there are few blocks
template <int DC>
__global__ __launch_bounds__(64 * kWaves) void attn_combine_kernel(CombineArgs a, int D) {
  constexpr int kLS = DC / 4;                // lanes per split row (float4 each)
  constexpr int kSPW = 64 / kLS;             // split rows per wave per load
  constexpr int kU = kPass / (kWaves * kSPW);  // loads per lane per pass
  static_assert(kLS == 4 || kLS == 8, "split rows are the lanes congruent mod kLS");
  __shared__ float4 red[kWaves][kLS];
  __shared__ float2 wml[kWaves];
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int sub = lane / kLS, dl = lane % kLS;
  const int row = blockIdx.x;
  const int d0 = blockIdx.y * DC;
  const int unit = blockIdx.z;  // s * H_kv + h
  // partials of this sequence: all num_splits slots, or after a suffix pass
  // shared out by length the prefix splits and the sequence's own share
  int ns = a.num_splits;
  if (a.bal_units > 0) {
    // (one-launch cascade: the prefix's units first, the same integer the
    // partial kernel computed)
    const int n_pre = a.prefix_tiles > 0 ? cascade_prefix_units(a.seq_lens, a.n_seqs, a.tok_begin, a.max_tiles,
                                                                a.bal_units, a.prefix_tiles, a.prefix_weight16,
                                                                a.min_prefix_units, lane)
                                         : a.prefix_splits;
    int n_t, W_t, O_t;
    bal_share(a.seq_lens, a.n_seqs, a.tok_begin, a.max_tiles, a.prefix_tiles > 0 ? a.bal_units - n_pre : a.bal_units,
              lane, n_t, W_t, O_t);
    ns = n_pre + __builtin_amdgcn_readfirstlane(__shfl(W_t, unit / a.H_kv));
  }
  const size_t base = static_cast<size_t>(unit) * a.num_splits;
  const size_t ostride4 = static_cast<size_t>(a.rows) * D / 4;  // float4s between consecutive splits
  const float4* o4 = reinterpret_cast<const float4*>(a.ws_o + (base * a.rows + row) * D + d0);
  const float2* ml2 = reinterpret_cast<const float2*>(a.ws_ml) + base * a.rows + row;
  const int s = unit / a.H_kv, h = unit % a.H_kv;
  const int jq = row / a.G, g = row % a.G;
  const size_t head = (static_cast<size_t>(s) * a.q_len + jq) * a.H_q + h * a.G + g;
  // the gate is read in the same round trip as the partials (unconditionally:
  // without a gate the load reads the output row, and the value is unused)
  const uint2 gw = *reinterpret_cast<const uint2*>(
      a.gate ? a.gate + head * a.gate_hstride + d0 + 4 * (tid % kLS) : a.out + head * D + d0 + 4 * (tid % kLS));

  // this wave's running merge: maximum M, sum of weighted l (per split row,
  // summed over the rows at the end) and of weighted o
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  float M = -INFINITY;
  float lsum = 0.f;
  for (int p0 = 0; p0 < ns; p0 += kPass) {
    // issue every load of this pass first (unconditional, the index clamped
    // to the last partial: a load under a branch would make the compiler
    // wait for each one in turn); the kLS lanes of a split row read the same
    // (m, l) pair
    float4 ov[kU];
    float2 mlv[kU];
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      const int i = min(p0 + (u * kWaves + wave) * kSPW + sub, ns - 1);
      ov[u] = o4[i * ostride4 + dl];
      mlv[u] = ml2[static_cast<size_t>(i) * a.rows];
    }
    float mi[kU];
    float mp = -INFINITY;
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      const bool in = p0 + (u * kWaves + wave) * kSPW + sub < ns;  // past the partials: weight 0
      mi[u] = in ? mlv[u].x : -INFINITY;
      mp = fmaxf(mp, mi[u]);
    }
    mp = max_rows<kLS>(mp);
    const float M_new = fmaxf(M, mp);
    const float Ms = (M_new == -INFINITY) ? 0.f : M_new;
    const float rescale = (M == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(M - Ms);
    acc.x *= rescale; acc.y *= rescale; acc.z *= rescale; acc.w *= rescale;
    lsum *= rescale;
    M = M_new;
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      // (v_exp_f32: a weight below 2^-126 of the maximum flushes to 0)
      const float w = (mi[u] == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(mi[u] - Ms);
      lsum += w * mlv[u].y;
      acc.x += w * ov[u].x; acc.y += w * ov[u].y; acc.z += w * ov[u].z; acc.w += w * ov[u].w;
    }
  }
  // sum over the split rows of the wave, then merge the waves
  acc.x = sum_rows<kLS>(acc.x); acc.y = sum_rows<kLS>(acc.y);
  acc.z = sum_rows<kLS>(acc.z); acc.w = sum_rows<kLS>(acc.w);
  lsum = sum_rows<kLS>(lsum);
  if (sub == 0) red[wave][dl] = acc;
  if (lane == 0) wml[wave] = make_float2(M, lsum);
  __syncthreads();
  if (tid < kLS) {
    float Mt = -INFINITY;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) Mt = fmaxf(Mt, wml[w].x);
    const float Ms = (Mt == -INFINITY) ? 0.f : Mt;
    float4 t = make_float4(0.f, 0.f, 0.f, 0.f);
    float l = 0.f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      const float c = (wml[w].x == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(wml[w].x - Ms);
      const float4 r4 = red[w][tid];
      t.x += c * r4.x; t.y += c * r4.y; t.z += c * r4.z; t.w += c * r4.w;
      l += c * wml[w].y;
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
  // 16-dim slices while 32-dim ones would leave most CUs idle (8 rows of
  // one sequence: 64 blocks), 32-dim ones otherwise (64 rows at 16-dim
  // slices, 1024 blocks, merged 25 % slower)
  const int64_t blocks32 = static_cast<int64_t>(a.rows) * (head_dim / 32) * a.n_seqs * a.H_kv;
  if (blocks32 < 256)
    hipLaunchKernelGGL(attn_combine_kernel<16>, dim3(a.rows, head_dim / 16, a.n_seqs * a.H_kv), dim3(64 * kWaves), 0,
                       stream, a, head_dim);
  else
    hipLaunchKernelGGL(attn_combine_kernel<32>, dim3(a.rows, head_dim / 32, a.n_seqs * a.H_kv), dim3(64 * kWaves), 0,
                       stream, a, head_dim);
  return hipGetLastError();
}

}  // namespace had
