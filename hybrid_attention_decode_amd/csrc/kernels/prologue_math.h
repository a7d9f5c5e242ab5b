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
// fp32; the result is rounded to bf16 (nearest even).  The host passes the
// exponent coefficient c = -2 log2(base) / R, so the frequency of pair i is
// exp2(i * c) with no fp64 logarithm or division on the device.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <cmath>

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

// Exponent coefficient of the rotation frequencies, -2 log2(base) / R
// (host side; 0 when nothing rotates).
inline double rope_coef(double base, int R) { return R > 0 ? -2.0 * std::log2(base) / R : 0.0; }

// cos and sin of the rotation angle pos * 2^(i c), c = rope_coef(base, R):
// the angle in fp64, reduced to [-pi, pi] in fp64 (multiplication by 1/(2 pi)
// and one fused multiply-add), then an fp32 sine and cosine.
__device__ __forceinline__ void rope_cs(int pos, int i, double coef, float& c, float& s) {
  const double inv_freq = exp2(static_cast<double>(i) * coef);
  const double theta = static_cast<double>(pos) * inv_freq;
  const double two_pi = 6.283185307179586476925286766559;
  const double inv_two_pi = 0.15915494309189533576888376337251;
  const double red = fma(-two_pi, rint(theta * inv_two_pi), theta);
  sincosf(static_cast<float>(red), &s, &c);
}

// RMSNorm * w, then the partial rotation with the given cos / sin of each
// of this lane's elements (1 and 0 past R).  The rotation partner of
// element d = l + 64 m is d +- R/2: in this lane's own registers when R/2 is
// a multiple of 64, in lane l ^ 32 (l ^ 16) when R/2 = 32 (16), reached by a
// lane swap; other R go through xrow, a D-float LDS row private to the
// calling wave.  The sums and products are the same in every case, so the
// result does not depend on how the partner is fetched.
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
  // sum over the wave: inside each 16-lane row by DPP (quad pairs, quad
  // halves, the other quad of 8, the other 8 of 16), then across the rows
  // (lanes l ^ 16, l ^ 32; a sum of two terms, in either order)
  ss += dpp<DPP_QUAD_XOR1>(ss);
  ss += dpp<DPP_QUAD_XOR2>(ss);
  ss += dpp<DPP_ROW_HALF_MIRROR>(ss);
  ss += dpp<DPP_ROW_ROR8>(ss);
  ss = sum_xor16(ss);
  ss = sum_xor32(ss);
  const float inv = 1.f / sqrtf(ss / static_cast<float>(D) + eps);
#pragma unroll
  for (int m = 0; m < E; ++m) x[m] = x[m] * inv * in.w[m];
  float other[E];
  const bool in_lane = half % 64 == 0, swap32 = half == 32, swap16 = half == 16;  // (uniform)
  if (in_lane) {
    const int hm = half / 64;
#pragma unroll
    for (int m = 0; m < E; ++m) {
      const int d = lane + 64 * m;
      other[m] = 0.f;
#pragma unroll
      for (int n = 0; n < E; ++n)  // x[m + hm] below R/2, x[m - hm] above (a constant index each way)
        if (n == m + hm || n == m - hm) other[m] = (d < half) == (n > m) ? x[n] : other[m];
    }
  } else if (swap32 || swap16) {
#pragma unroll
    for (int m = 0; m < E; ++m) {
      const auto p = swap32 ? __builtin_amdgcn_permlane32_swap(__float_as_uint(x[m]), __float_as_uint(x[m]), false, false)
                            : __builtin_amdgcn_permlane16_swap(__float_as_uint(x[m]), __float_as_uint(x[m]), false, false);
      // the two results hold x[m] of this lane and of its partner, in either order
      const float a = __uint_as_float(p[0]), b = __uint_as_float(p[1]);
      other[m] = __float_as_uint(a) == __float_as_uint(x[m]) ? b : a;
    }
  } else {
#pragma unroll
    for (int m = 0; m < E; ++m) xrow[lane + 64 * m] = x[m];
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
#pragma unroll
    for (int m = 0; m < E; ++m) {
      const int d = lane + 64 * m;
      other[m] = d < R ? xrow[d < half ? d + half : d - half] : 0.f;
    }
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
  }
#pragma unroll
  for (int m = 0; m < E; ++m) {
    const int d = lane + 64 * m;
    float r = x[m];
    if (d < R) r = d < half ? x[m] * cs[m] - other[m] * sn[m] : x[m] * cs[m] + other[m] * sn[m];
    y[m] = f32_to_bf16(r);
  }
}

// The same, forming this row's angles at `pos` itself (coef = rope_coef).
template <int D>
__device__ __forceinline__ void row_norm_rope(const RowIn<D>& in, int pos, int R, double coef, float eps, float* xrow,
                                              int lane, uint16_t (&y)[D / 64]) {
  constexpr int E = D / 64;
  const int half = R / 2;
  float cs[E], sn[E];
#pragma unroll
  for (int m = 0; m < E; ++m) {
    const int d = lane + 64 * m;
    cs[m] = 1.f;
    sn[m] = 0.f;
    if (64 * m < R && d < R) rope_cs(pos, d % half, coef, cs[m], sn[m]);
  }
  row_norm_rope_cs<D>(in, cs, sn, R, eps, xrow, lane, y);
}

}  // namespace had
