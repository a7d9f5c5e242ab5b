// Per-row arithmetic of the fused attention prologue, shared by the
// stand-alone prologue kernel and the attention kernels that run it inline,
// so every path produces the same bits (zubnet.ai TokenSpeed article, second
// paragraph: QK-RMSNorm, partial RoPE and the gate split fused into one
// kernel with intermediates in registers).
//
// One wave owns one D-long row; lane l holds elements d = l + 64 m.
//   RMSNorm(x) = x / sqrt(mean(x^2) + eps) * w          (fp32; Zhang & Sennrich 2019)
//   dims d < R rotate in pairs (i, i + R/2), angle pos * base^(-2i/R):
//     y_i' = y_i cos - y_{i+R/2} sin,  y_{i+R/2}' = y_{i+R/2} cos + y_i sin
//   (rotary embedding, Su et al. RoFormer 2021, on a prefix of the head).
// The angle is formed in fp64 (at pos ~ 1e6 an fp32 product is off by
// ~0.06 rad), reduced to [-pi, pi] in fp64, and its sine and cosine taken in
// fp32; the result is rounded to bf16 (nearest even).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kcommon.h"

namespace had {

template <int D>
struct RowIn {
  uint16_t x[D / 64];  // raw bf16 row elements of this lane
  float w[D / 64];     // norm weights of those elements
};

// Issue the loads of one row and its weights (kept apart from the
// arithmetic so callers can put them ahead of other memory traffic).
template <int D>
__device__ __forceinline__ void row_load(RowIn<D>& in, const uint16_t* __restrict__ src, const float* __restrict__ w,
                                         int lane) {
#pragma unroll
  for (int m = 0; m < D / 64; ++m) {
    in.x[m] = src[lane + 64 * m];
    in.w[m] = w[lane + 64 * m];
  }
}

// The row elements only (rows that share their weights with a loaded row).
template <int D>
__device__ __forceinline__ void row_load_x(RowIn<D>& in, const uint16_t* __restrict__ src, int lane) {
#pragma unroll
  for (int m = 0; m < D / 64; ++m) in.x[m] = src[lane + 64 * m];
}

// cos and sin of the rotation angle pos * base^(-2i/R): the angle in fp64,
// reduced to [-pi, pi] in fp64, then an fp32 sine and cosine.
__device__ __forceinline__ void rope_cs(int pos, int i, int R, double log2_base, float& c, float& s) {
  const double inv_freq = exp2(-2.0 * i / R * log2_base);
  const double theta = static_cast<double>(pos) * inv_freq;
  const double two_pi = 6.283185307179586476925286766559;
  const double red = theta - two_pi * rint(theta / two_pi);
  sincosf(static_cast<float>(red), &s, &c);
}

// RMSNorm * w, then the partial rotation with the given cos / sin of each
// of this lane's elements (1 and 0 past R); xrow is a D-float LDS row
// private to the calling wave (used to fetch rotation partners).
template <int D>
__device__ __forceinline__ void row_norm_rope_cs(const RowIn<D>& in, const float (&cs)[D / 64],
                                                 const float (&sn)[D / 64], int R, float eps, float* xrow, int lane,
                                                 uint16_t (&y)[D / 64]) {
  constexpr int E = D / 64;
  const int half = R / 2;
  float x[E];
  float ss = 0.f;
#pragma unroll
  for (int m = 0; m < E; ++m) {
    x[m] = bf16_to_f32(in.x[m]);
    ss += x[m] * x[m];
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) ss += shfl_xor_f(ss, off);
  const float inv = 1.f / sqrtf(ss / static_cast<float>(D) + eps);
#pragma unroll
  for (int m = 0; m < E; ++m) {
    x[m] = x[m] * inv * in.w[m];
    xrow[lane + 64 * m] = x[m];
  }
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
#pragma unroll
  for (int m = 0; m < E; ++m) {
    const int d = lane + 64 * m;
    float r = x[m];
    if (d < R) {
      const float other = xrow[d < half ? d + half : d - half];
      r = d < half ? x[m] * cs[m] - other * sn[m] : x[m] * cs[m] + other * sn[m];
    }
    y[m] = f32_to_bf16(r);
  }
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
}

// The same, forming this row's angles at `pos` itself.
template <int D>
__device__ __forceinline__ void row_norm_rope(const RowIn<D>& in, int pos, int R, double base, float eps, float* xrow,
                                              int lane, uint16_t (&y)[D / 64]) {
  constexpr int E = D / 64;
  const int half = R / 2;
  const double log2_base = log2(base);
  float cs[E], sn[E];
#pragma unroll
  for (int m = 0; m < E; ++m) {
    const int d = lane + 64 * m;
    cs[m] = 1.f;
    sn[m] = 0.f;
    if (d < R) rope_cs(pos, d % half, R, log2_base, cs[m], sn[m]);
  }
  row_norm_rope_cs<D>(in, cs, sn, R, eps, xrow, lane, y);
}

}  // namespace had
