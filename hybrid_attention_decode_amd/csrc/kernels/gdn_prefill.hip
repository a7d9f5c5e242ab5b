// Gated delta rule over whole prompts, chunk-parallel (GDN prefill).
//
// For one (sequence, head), a chunk of C = 64 tokens starting from state S0
// (d_v x d_k), with g_t = log alpha_t, lg_t = sum_{i<=t} g_i and
// gamma_t = exp(lg_t) inside the chunk, the delta-rule inputs u_t
// (S_t = alpha_t S_{t-1} + u_t k_t^T) satisfy
//   (I + A) U = diag(beta) (V - diag(gamma) K S0^T),
//   A[t][i] = beta_t exp(lg_t - lg_i) k_t.k_i  (i < t, else 0),
// so with T = (I + A)^-1 (unit lower triangular)
//   U  = U' - W S0^T,   U' = T diag(beta) V,   W = T diag(beta gamma) K,
//   o  = diag(gamma) Q S0^T + Aqk U,   Aqk[t][i] = exp(lg_t - lg_i) q_t.k_i (i <= t),
//   S_C = gamma_C S0 + (diag(gamma_C / gamma) U)^T K.
// (WY / UT form of the delta rule: Yang et al., NeurIPS 2024, "Parallelizing
// Linear Transformers with the Delta Rule over Sequence Length"; the gated
// recurrence of the Gated DeltaNet paper, Yang, Kautz & Hatamizadeh, ICLR
// 2025.  GDN layers of the hybrid model: 24-ai.news TokenSpeed article.)
//
// Two kernels (and a link kernel between two scan passes for long prompts):
//  * prep, one workgroup per (sequence, chunk, head), all chunks at once:
//    K K^T and K Q^T on MFMA, the triangular solve by forward substitution
//    (one wave, lane j = column j of T, fp32), then U' and W on MFMA.  The
//    results go to the workspace already in the register layout of the scan
//    kernel's MFMA operands.
//  * scan, one workgroup of 4 waves per (sequence, head, 16 rows of S): the
//    state slice stays in registers across the chunks of the sequence; wave
//    w owns the chunk's tokens 16w .. 16w+15 for U and the output and the
//    state columns 32w .. 32w+31 for the update.  Two barriers per chunk
//    exchange U and the new state through LDS.  The chunk's output columns
//    of the slice, o = q_scale (diag(gamma) Q S0^T + Aqk U), are formed
//    while S0 and U are at hand (Q read from the input, Aqk from the
//    workspace), so neither U nor the chunk states go back to memory.
// Products with a fp32 operand (the state, T, W, Aqk, U) use the split
// x = hi + lo of both bf16 halves (hi*hi + hi*lo + lo*hi, or two terms when
// the other operand is exact bf16), so each product keeps ~16 mantissa bits.
//
// MFMA v_mfma_f32_16x16x32_bf16 operand layout: lane (r, g), r = lane % 16,
// g = lane / 16, holds A[row r][k = 8g .. 8g+7] and B[k = 8g .. 8g+7][col r];
// the result lane (r, g) holds C[rows 4g .. 4g+3][col r].  A contraction may
// take its k index in any order both operands agree on: the scan kernel
// contracts over d_k in the order sigma(ks, g, j) = 32 ks + 16 (j / 4) + 4 g
// + j % 4 and over tokens in the same order tau(ks', g, j) -- the order in
// which a result tile pair (16 x 16 tiles 2 ks and 2 ks + 1) leaves each
// lane -- so results feed the next product without any reshuffle.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>

#include "../host/status.h"
#include "had.h"
#include "kcommon.h"

using had::fail;

namespace had {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

constexpr int kC = 64;  // tokens per chunk

__device__ __forceinline__ f32x4_t mfma(u32x4_t a, u32x4_t b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a), __builtin_bit_cast(bf16x8_t, b), c,
                                                 0, 0, 0);
}

// x -> hi = bf16(x), lo = bf16(x - hi), both round to nearest even.
__device__ __forceinline__ void split8(const float (&x)[8], u32x4_t& hi, u32x4_t& lo) {
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const uint32_t h = pack_bf16x2(x[2 * j], x[2 * j + 1]);
    hi[j] = h;
    lo[j] = pack_bf16x2(x[2 * j] - bf16_lo(h), x[2 * j + 1] - bf16_hi(h));
  }
}

__device__ __forceinline__ void cat8(f32x4_t a, f32x4_t b, float (&x)[8]) {
  x[0] = a[0]; x[1] = a[1]; x[2] = a[2]; x[3] = a[3];
  x[4] = b[0]; x[5] = b[1]; x[6] = b[2]; x[7] = b[3];
}

// Workspace block of one (sequence, chunk, head), in 16-byte units; every
// array is [..][64 lanes] in the scan kernel's operand layout.
template <int DK, int DV>
struct PL {
  static constexpr int KS = DK / 32;             // k-steps over d_k
  static constexpr int DT = DK / 16;             // d_k tiles
  static constexpr int VT = DV / 16;             // d_v tiles
  static constexpr int W_HI = 0;                 // W, A operand: [t-tile][ks][lane], d_k in sigma order
  static constexpr int W_LO = W_HI + 4 * KS * 64;
  static constexpr int UP = W_LO + 4 * KS * 64;  // U' (U after the scan), result layout: [t-tile][v-tile][lane]
  static constexpr int A_HI = UP + 4 * VT * 64;  // Aqk, A operand: [t-tile][ks'][lane], tokens in tau order
  static constexpr int A_LO = A_HI + 4 * 2 * 64;
  static constexpr int KT = A_LO + 4 * 2 * 64;   // K^T, A operand: [d_k tile][ks'][lane], tokens in tau order
  static constexpr int GAM = KT + DT * 2 * 64;   // 64 floats gamma_t, then 64 floats gamma_C / gamma_t
  static constexpr int TOTAL = GAM + 2 * kC / 4;
};

struct PrefillArgs {
  float* pool;
  const int32_t* in_idx;
  const int32_t* out_idx;
  const int32_t* cu;
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  const float* alpha;
  const float* beta;
  float* o;
  u32x4_t* ws;
  int32_t* d_err;
  int n_seqs, H, n_slots, max_len, max_chunks, raw_gates;
  float q_scale;
  // segmented scan: the chunks of a sequence in n_segs runs of seg_chunks
  // (the last may be shorter or empty); seg: per (sequence, segment, head)
  // the fp32 blocks of SegL; phase 0 = one pass, 1 / 3 = the two scan
  // passes of the segmented form (phase 2 is the link kernel)
  float* seg;
  int n_segs, seg_chunks, phase;
};

// Per (sequence, segment, head), fp32 [row][d_k] blocks of the segmented
// scan: PI = the segment's transition (the state after the segment is
// S_start PI + SE), SE = the state the segment reaches from zero, SS = the
// state the segment starts from.
template <int DK, int DV>
struct SegL {
  static constexpr size_t PI = 0;
  static constexpr size_t SE = static_cast<size_t>(DK) * DK;
  static constexpr size_t SS = SE + static_cast<size_t>(DV) * DK;
  static constexpr size_t TOTAL = SS + static_cast<size_t>(DV) * DK;
};

// One 16-byte piece of a bf16 row (zeros for rows past the chunk).
// 16 bytes at src of token row t of the chunk (zero past its n tokens); the
// address is clamped to the chunk's last token, so the load is unconditional
// (loads of a thread batch up instead of each waiting behind a branch) and
// stays inside the input
__device__ __forceinline__ u32x4_t row16(const uint16_t* src, size_t stride, int base, int t, int n) {
  const u32x4_t r = *reinterpret_cast<const u32x4_t*>(src + static_cast<size_t>(base + min(t, n - 1)) * stride);
  return t < n ? r : u32x4_t{0u, 0u, 0u, 0u};
}

template <int DK, int DV>
__global__ __launch_bounds__(256) void gdn_prefill_prep_kernel(PrefillArgs a) {
  using L = PL<DK, DV>;
  constexpr int KS = L::KS, DT = L::DT, VT = L::VT;
  const int c = blockIdx.x, h = blockIdx.y, s = blockIdx.z;
  const int tok0 = a.cu[s], len = a.cu[s + 1] - tok0;
  if (tok0 < 0 || len < 0 || len > a.max_len) return;  // reported by the scan kernel
  const int n = min(kC, len - c * kC);                  // tokens of this chunk
  if (n <= 0) return;
  const int base = tok0 + c * kC;
  u32x4_t* ws = a.ws + ((static_cast<size_t>(s) * a.max_chunks + c) * a.H + h) * L::TOTAL;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63, r16 = lane & 15, g = lane >> 4;
  const size_t rstride = static_cast<size_t>(a.H) * DK;  // between tokens of q / k

  __shared__ float lgL[kC], betaL[kC];
  __shared__ __align__(16) uint16_t ktL[DK][kC + 8];  // K^T [d][token]
  __shared__ __align__(16) uint16_t vtL[DV][kC + 8];  // V^T [d][token]
  __shared__ __align__(16) float amat[kC][kC + 4];    // A, then T diag(beta)
  __shared__ __align__(16) float tbg[kC][kC + 4];     // T diag(beta gamma)

  // K^T and V^T into LDS: an item is (token pair p, 8 dims dc); two 16-byte
  // rows transpose into 8 words of (token 2p, token 2p+1) at one dim.  A
  // thread holds DD / 64 items of each; all their loads, and those of the
  // K operand rows below, are in flight before the first LDS write.
  constexpr int NKI = DK / 64, NVI = DV / 64;
  const size_t vstride = static_cast<size_t>(a.H) * DV;
  u32x4_t sk[NKI][2], sv[NVI][2];
#pragma unroll
  for (int j = 0; j < NKI; ++j) {
    const int it = threadIdx.x + 256 * j, p = it & 31, dc = it >> 5;
#pragma unroll
    for (int e = 0; e < 2; ++e) sk[j][e] = row16(a.k + h * DK + 8 * dc, rstride, base, 2 * p + e, n);
  }
#pragma unroll
  for (int j = 0; j < NVI; ++j) {
    const int it = threadIdx.x + 256 * j, p = it & 31, dc = it >> 5;
#pragma unroll
    for (int e = 0; e < 2; ++e) sv[j][e] = row16(a.v + h * DV + 8 * dc, vstride, base, 2 * p + e, n);
  }
  // K rows of the four token tiles as MFMA operands (zero past the chunk),
  // and this wave's own tile once more for A (a register copy indexed by the
  // wave would compile to selects)
  u32x4_t kr[4][KS], kown[KS];
#pragma unroll
  for (int tt = 0; tt < 4; ++tt) {
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) kr[tt][ks] = row16(a.k + h * DK + 32 * ks + 8 * g, rstride, base, 16 * tt + r16, n);
  }
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) kown[ks] = row16(a.k + h * DK + 32 * ks + 8 * g, rstride, base, 16 * wave + r16, n);
  // gates (after the loads above are issued, so wave 0's round trip for
  // them overlaps the rest): lg = inclusive prefix sum of log alpha (0 past
  // the chunk), beta
  if (wave == 0) {
    float la = 0.f, be = 0.f;
    if (lane < n) {
      const size_t th = static_cast<size_t>(base + lane) * a.H + h;
      const float al = a.alpha[th];
      be = a.beta[th];
      if (a.raw_gates) {
        la = al;
        be = 1.f / (1.f + expf(-be));
      } else {
        la = logf(al);
      }
    }
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const float y = __shfl_up(la, off);
      if (lane >= off) la += y;
    }
    lgL[lane] = la;
    betaL[lane] = be;
    const float lgC = __shfl(la, 63);
    float* gw = reinterpret_cast<float*>(ws + L::GAM);
    gw[lane] = expf(la);
    gw[kC + lane] = expf(lgC - la);
  }

  auto put_t = [&](const u32x4_t& x0, const u32x4_t& x1, int it, uint16_t* dst) {
    const int p = it & 31, dc = it >> 5, t0 = 2 * p;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      // dims 8dc + 2j (low halves) and 8dc + 2j + 1 (high halves)
      *reinterpret_cast<uint32_t*>(dst + (8 * dc + 2 * j) * (kC + 8) + t0) = perm_b32(x1[j], x0[j], 0x05040100u);
      *reinterpret_cast<uint32_t*>(dst + (8 * dc + 2 * j + 1) * (kC + 8) + t0) = perm_b32(x1[j], x0[j], 0x07060302u);
    }
  };
#pragma unroll
  for (int j = 0; j < NKI; ++j) put_t(sk[j][0], sk[j][1], threadIdx.x + 256 * j, &ktL[0][0]);
#pragma unroll
  for (int j = 0; j < NVI; ++j) put_t(sv[j][0], sv[j][1], threadIdx.x + 256 * j, &vtL[0][0]);
  __syncthreads();

  // A (strictly lower): wave w forms the tiles of token rows 16w .. 16w+15
  {
#pragma unroll
    for (int nt = 0; nt < 4; ++nt) {
      if (nt > wave) break;
      f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) acc = mfma(kown[ks], kr[nt][ks], acc);
      const int i = 16 * nt + r16;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int tr = 16 * wave + 4 * g + r;
        amat[tr][i] = i < tr ? betaL[tr] * expf(lgL[tr] - lgL[i]) * acc[r] : 0.f;
      }
    }
  }
  __syncthreads();

  if (wave == 0) {
    // T = (I + A)^-1 by forward substitution; lane j computes column j:
    // T[t][j] = [t == j] - sum_{i<t} A[t][i] T[i][j]
    // Row t + 1 of A is read while row t is reduced (two register rows), so
    // the LDS latency overlaps the arithmetic instead of following each read.
    float x[kC], ra[kC], rb[kC];
    auto load_row = [&](int t, float (&r)[kC]) {
#pragma unroll
      for (int i4 = 0; i4 < t; i4 += 4) {
        const float4 av = *reinterpret_cast<const float4*>(&amat[t][i4]);
        r[i4] = av.x;
        r[i4 + 1] = av.y;
        r[i4 + 2] = av.z;
        r[i4 + 3] = av.w;
      }
    };
    x[0] = lane == 0 ? 1.f : 0.f;
    load_row(1, ra);
#pragma unroll
    for (int t = 1; t < kC; ++t) {
      float(&cur)[kC] = (t & 1) ? ra : rb;
      float(&nxt)[kC] = (t & 1) ? rb : ra;
      if (t + 1 < kC) load_row(t + 1, nxt);
      __builtin_amdgcn_sched_barrier(0);
      float acc[4] = {t == lane ? 1.f : 0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int i = 0; i < t; ++i) acc[i & 3] = fmaf(-cur[i], x[i], acc[i & 3]);
      x[t] = (acc[0] + acc[1]) + (acc[2] + acc[3]);
    }
    const float bj = betaL[lane], bgj = bj * expf(lgL[lane]);
#pragma unroll
    for (int t = 0; t < kC; ++t) {
      amat[t][lane] = x[t] * bj;  // the wave's reads of A are done: T diag(beta) takes its place
      tbg[t][lane] = x[t] * bgj;
    }
  } else {
    // Aqk for the scan kernel: tile (i-tile it, t-tile tt) of (K Q^T) leaves
    // lane (t, g) holding i = 16 it + 4g + r, so tiles 2ks' and 2ks'+1 give
    // the A operand of token step ks' in tau order
    for (int tt = wave - 1; tt < 4; tt += 3) {
      const int t = 16 * tt + r16;
      u32x4_t qr[KS];
#pragma unroll
      for (int ks = 0; ks < KS; ++ks)
        qr[ks] = row16(a.q + h * DK + 32 * ks + 8 * g, rstride, base, t, n);
      float e[4][4];
#pragma unroll
      for (int it = 0; it < 4; ++it) {
        f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
        if (it <= tt) {
#pragma unroll
          for (int ks = 0; ks < KS; ++ks) acc = mfma(kr[it][ks], qr[ks], acc);
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int i = 16 * it + 4 * g + r;
          e[it][r] = i <= t ? expf(lgL[t] - lgL[i]) * acc[r] : 0.f;
        }
      }
#pragma unroll
      for (int kp = 0; kp < 2; ++kp) {
        const float x8[8] = {e[2 * kp][0], e[2 * kp][1], e[2 * kp][2], e[2 * kp][3],
                             e[2 * kp + 1][0], e[2 * kp + 1][1], e[2 * kp + 1][2], e[2 * kp + 1][3]};
        u32x4_t hi, lo;
        split8(x8, hi, lo);
        ws[L::A_HI + (tt * 2 + kp) * 64 + lane] = hi;
        ws[L::A_LO + (tt * 2 + kp) * 64 + lane] = lo;
      }
    }
    // K^T for the state update: lane (dk, g) of (d_k tile dt, token step
    // ks') holds tokens 32ks' + 4g .. +3 and 32ks' + 16 + 4g .. +3
    for (int b = wave - 1; b < DT * 2; b += 3) {
      const int dt = b >> 1, kp = b & 1;
      const uint16_t* row = &ktL[16 * dt + r16][32 * kp + 4 * g];
      const uint2 x0 = *reinterpret_cast<const uint2*>(row);
      const uint2 x1 = *reinterpret_cast<const uint2*>(row + 16);
      ws[L::KT + b * 64 + lane] = u32x4_t{x0.x, x0.y, x1.x, x1.y};
    }
  }
  __syncthreads();

  // U' = T diag(beta) V and W = T diag(beta gamma) K for token rows 16w ..
  {
    const int t = 16 * wave + r16;
    u32x4_t tbh[2], tbl[2], tgh[2], tgl[2];
#pragma unroll
    for (int kp = 0; kp < 2; ++kp) {
      float x8[8];
      cat8(*reinterpret_cast<const f32x4_t*>(&amat[t][32 * kp + 8 * g]),
           *reinterpret_cast<const f32x4_t*>(&amat[t][32 * kp + 8 * g + 4]), x8);
      split8(x8, tbh[kp], tbl[kp]);
      cat8(*reinterpret_cast<const f32x4_t*>(&tbg[t][32 * kp + 8 * g]),
           *reinterpret_cast<const f32x4_t*>(&tbg[t][32 * kp + 8 * g + 4]), x8);
      split8(x8, tgh[kp], tgl[kp]);
    }
#pragma unroll
    for (int vt = 0; vt < VT; ++vt) {
      f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kp = 0; kp < 2; ++kp) {
        const u32x4_t b = *reinterpret_cast<const u32x4_t*>(&vtL[16 * vt + r16][32 * kp + 8 * g]);
        acc = mfma(tbh[kp], b, acc);
        acc = mfma(tbl[kp], b, acc);
      }
      ws[L::UP + (wave * VT + vt) * 64 + lane] = __builtin_bit_cast(u32x4_t, acc);
    }
    // W^T = K^T (T diag(beta gamma))^T: tile (d_k tile dt, t-tile w) leaves
    // lane (t, g) holding d_k = 16 dt + 4g + r, so tiles 2ks and 2ks+1 give
    // the A operand of d_k step ks in sigma order
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      f32x4_t cw[2];
#pragma unroll
      for (int e = 0; e < 2; ++e) {
        const int dt = 2 * ks + e;
        f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kp = 0; kp < 2; ++kp) {
          const u32x4_t am = *reinterpret_cast<const u32x4_t*>(&ktL[16 * dt + r16][32 * kp + 8 * g]);
          acc = mfma(am, tgh[kp], acc);
          acc = mfma(am, tgl[kp], acc);
        }
        cw[e] = acc;
      }
      float x8[8];
      cat8(cw[0], cw[1], x8);
      u32x4_t hi, lo;
      split8(x8, hi, lo);
      ws[L::W_HI + (wave * KS + ks) * 64 + lane] = hi;
      ws[L::W_LO + (wave * KS + ks) * 64 + lane] = lo;
    }
  }
}

// Scan over the chunks of one (sequence, head) for state rows 16 vs .. +15:
// what the state needs (W, K^T, U') is on this sequential path; the pass
// that emits the output (EMIT) also reads Q and Aqk, one chunk ahead like
// the rest, and writes the chunk's output columns of the slice.
//
// Segmented form (a long prompt with few heads: one pass would keep only
// units x d_v/16 workgroups busy along a chain of every chunk).  With
// S_{c+1} = S_c A_c + B_c per chunk, a run of chunks maps its start state
// S to S PI + SE, PI = prod A_c (d_k x d_k) and SE the state reached from
// zero.  Phase 1 scans every segment but the last at once, twice over: the
// d_v state rows from zero (giving SE; the first segment starts from the
// input state instead, so its SE is the second segment's start state) and,
// past the first segment, the d_k rows of the identity with U' = 0 (giving
// PI), storing nothing per chunk; the link kernel chains the segments'
// start states; phase 3 is the one-pass scan again, every segment at once
// from its start state, emitting the output.
template <int DK, int DV, bool EMIT>
__global__ __launch_bounds__(256, 2) void gdn_prefill_scan_kernel(PrefillArgs a) {
  using L = PL<DK, DV>;
  using G = SegL<DK, DV>;
  constexpr int KS = L::KS, VT = L::VT, DT = L::DT;
  // block -> (item = (s * H + h) * n_segs + segment, slice): the slices of
  // one item share the item's workspace blocks, so they go to one XCD
  // (blocks are dealt to the 8 XCDs round robin).  Phase 1 has VT slices of
  // state rows and DT of transition rows.
  const int NSL = a.phase == 1 ? VT + DT : VT;
  const int n_items_seg = a.phase == 1 ? a.n_segs - 1 : a.n_segs;  // phase 1 skips the last segment
  const int b = blockIdx.x;
  const int item = (b / 8 / NSL) * 8 + b % 8, vs = (b / 8) % NSL;
  if (item >= a.n_seqs * a.H * n_items_seg) return;
  const int seg = item % n_items_seg, unit = item / n_items_seg;
  const int s = unit / a.H, h = unit % a.H;
  const bool pi_rows = vs >= VT;            // phase 1: rows of the transition
  if (a.phase == 1 && pi_rows && seg == 0) return;  // the first segment's transition is not needed
  const int vsc = pi_rows ? VT - 1 : vs;    // (their U' loads read a real slice and are discarded)
  // (wave is made uniform so that tests on it are scalar branches)
  const int wave = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x) >> 6);
  const int lane = threadIdx.x & 63, r16 = lane & 15, g = lane >> 4;

  const int tok0 = a.cu[s], len = a.cu[s + 1] - tok0;
  const int in = a.in_idx[s], out = a.out_idx[s];
  const bool bad_len = tok0 < 0 || len < 0 || len > a.max_len;
  const bool bad_slot = in < -1 || in >= a.n_slots || out < 0 || out >= a.n_slots;
  if (bad_len || bad_slot) {
    if (threadIdx.x == 0 && vs == 0 && seg == 0)
      set_err(a.d_err, (bad_len ? HAD_DERR_SEQLEN : 0) | (bad_slot ? HAD_DERR_SLOT : 0));
    return;
  }
  // this block's chunks [c0, c1): the whole sequence, or its segment
  const int n_chunks = (len + kC - 1) / kC;
  const int c0 = min(seg * a.seg_chunks, n_chunks);
  const int c1 = a.n_segs > 1 ? min(c0 + a.seg_chunks, n_chunks) : n_chunks;
  const size_t slot_elems = static_cast<size_t>(a.H) * DV * DK;
  const size_t row_off = (static_cast<size_t>(h) * DV + 16 * vsc + r16) * DK;
  float* segb = a.seg + ((static_cast<size_t>(s) * a.n_segs + seg) * a.H + h) * G::TOTAL;

  __shared__ f32x4_t ubuf[4][64];         // U tiles of the chunk (result layout)
  __shared__ u32x4_t sbuf[KS][2][64];     // new state as B operands (hi, lo) per d_k step
  __shared__ __align__(16) float rbuf[kC];  // gamma_C / gamma_t of the chunk

  const int kw = wave < KS ? wave : 0;  // a wave that owns no d_k step (d_k 64) mirrors step 0 and discards it

  // state rows as B operands: lane (v, g) holds S[v][sigma(ks, g, j)]; the
  // wave's own d_k step also in fp32 (sown) and as its hi/lo pair (ohi, olo),
  // so that no register array is indexed by the wave number (a dynamic
  // index into registers compiles to a compare-and-select chain)
  u32x4_t shi[KS], slo[KS], ohi, olo;
  f32x4_t sown[2] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
  {
    // start state: the input slot (one pass), zero or the identity rows
    // (phase 1), the segment's start state (phase 3; the link kernel wrote
    // every segment's, the first included)
    const float* src = a.phase == 3 ? segb + G::SS + static_cast<size_t>(16 * vs + r16) * DK
                                    : a.pool + static_cast<size_t>(max(in, 0)) * slot_elems + row_off;
    const bool from_slot = a.phase == 0 || (a.phase == 1 && seg == 0 && !pi_rows);
    const bool zero = from_slot && in < 0;
    const int id_row = 16 * (vs - VT) + r16;  // phase 1, transition rows: row of the identity
    // columns col0 .. +3 and col0 + 16 .. +3 of this lane's row
    auto start = [&](int col0, f32x4_t& p0, f32x4_t& p1) {
      if (a.phase == 1 && !from_slot) {
        const float on = pi_rows ? 1.f : 0.f;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          p0[j] = (col0 + j == id_row) ? on : 0.f;
          p1[j] = (col0 + 16 + j == id_row) ? on : 0.f;
        }
      } else {
        p0 = *reinterpret_cast<const f32x4_t*>(src + col0);
        p1 = *reinterpret_cast<const f32x4_t*>(src + col0 + 16);
        if (zero) p0 = p1 = f32x4_t{0.f, 0.f, 0.f, 0.f};  // no input slot: zero state
      }
    };
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      f32x4_t p0, p1;
      start(32 * ks + 4 * g, p0, p1);
      float x8[8];
      cat8(p0, p1, x8);
      split8(x8, shi[ks], slo[ks]);
    }
    start(32 * kw + 4 * g, sown[0], sown[1]);
    float x8[8];
    cat8(sown[0], sown[1], x8);
    split8(x8, ohi, olo);
  }

  u32x4_t* blk0 = a.ws + static_cast<size_t>(s) * a.max_chunks * a.H * L::TOTAL + static_cast<size_t>(h) * L::TOTAL;

  // A chunk's operands, loaded one chunk ahead (none depends on the state).
  // Every load is unconditional: a load under a branch would make the join
  // wait for all loads in flight, the prefetch included.  Vector-memory
  // operations retire in issue order, and a store retires only when the
  // write is acknowledged (slow once the workspace spills to HBM), so the
  // step issues its stores after the next chunk's loads: waiting for those
  // loads then never waits for a store of the same step.
  struct Ops {
    u32x4_t whi[KS], wlo[KS], kt[2][2];
    f32x4_t up;
    float rat, gC;
  };
  auto load_w = [&](int c, Ops& p) {
    const u32x4_t* blk = blk0 + static_cast<size_t>(c) * a.H * L::TOTAL;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      p.whi[ks] = blk[L::W_HI + (wave * KS + ks) * 64 + lane];
      p.wlo[ks] = blk[L::W_LO + (wave * KS + ks) * 64 + lane];
    }
  };
  auto load_rest = [&](int c, Ops& p) {
    const u32x4_t* blk = blk0 + static_cast<size_t>(c) * a.H * L::TOTAL;
    const float* gw = reinterpret_cast<const float*>(blk + L::GAM);
    p.up = __builtin_bit_cast(f32x4_t, blk[L::UP + (wave * VT + vsc) * 64 + lane]);
    if (pi_rows) p.up = f32x4_t{0.f, 0.f, 0.f, 0.f};  // the transition: U' = 0
#pragma unroll
    for (int e = 0; e < 2; ++e)
#pragma unroll
      for (int kp = 0; kp < 2; ++kp) p.kt[e][kp] = blk[L::KT + ((2 * kw + e) * 2 + kp) * 64 + lane];
    p.rat = gw[kC + lane];
    p.gC = gw[kC - 1];
  };
  // The output's operands of one chunk (EMIT): Q rows 16w + r (d_k in sigma
  // order; rows past the sequence read its last row, their output is not
  // stored), the Aqk rows and gamma_t of this lane's output rows.  One
  // register set, refilled for the next chunk as soon as this chunk's
  // products have read it (a step ahead, the latency stays hidden).
  struct OutOps {
    u32x4_t qa[KS], ahi[2], alo[2];
    f32x4_t gam;
  };
  auto load_out = [&](int c, OutOps& p) {
    const u32x4_t* blk = blk0 + static_cast<size_t>(c) * a.H * L::TOTAL;
    const int tq = min(c * kC + 16 * wave + r16, len - 1);
    const uint16_t* qp = a.q + (static_cast<size_t>(tok0 + tq) * a.H + h) * DK;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const uint2 x0 = *reinterpret_cast<const uint2*>(qp + 32 * ks + 4 * g);
      const uint2 x1 = *reinterpret_cast<const uint2*>(qp + 32 * ks + 16 + 4 * g);
      p.qa[ks] = u32x4_t{x0.x, x0.y, x1.x, x1.y};
    }
    // Aqk rows of the wave: the second token step only for rows 32 .. 63 (it
    // holds zeros above); a zero-size descriptor returns zeros for waves 0
    // and 1 without a memory request, and no load sits under a branch
    constexpr int kAqk = L::A_LO + 4 * 2 * 64 - L::A_HI;  // 16-byte units of Aqk (hi, lo)
    const __amdgpu_buffer_rsrc_t ar0 =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<u32x4_t*>(blk + L::A_HI), 0, kAqk * 16, kBufferRsrcWord3);
    const __amdgpu_buffer_rsrc_t ar1 = __builtin_amdgcn_make_buffer_rsrc(const_cast<u32x4_t*>(blk + L::A_HI), 0,
                                                                         wave < 2 ? 0 : kAqk * 16, kBufferRsrcWord3);
#pragma unroll
    for (int kp = 0; kp < 2; ++kp) {
      const int off = ((wave * 2 + kp) * 64 + lane) * 16;
      p.ahi[kp] = __builtin_amdgcn_raw_buffer_load_b128(kp ? ar1 : ar0, off, 0, 0);
      p.alo[kp] = __builtin_amdgcn_raw_buffer_load_b128(kp ? ar1 : ar0, off + (L::A_LO - L::A_HI) * 16, 0, 0);
    }
    p.gam = *reinterpret_cast<const f32x4_t*>(reinterpret_cast<const float*>(blk + L::GAM) + 16 * wave + 4 * g);
  };

  // one chunk: c with operands p; the operands of chunk cn load into pn
  OutOps po;
  auto step = [&](int c, const Ops& p, int cn, Ops& pn) {
    if (wave == 0) rbuf[lane] = p.rat;
    // U = U' - W S0^T for token rows 16w .. (the split terms accumulate in
    // separate chains); chunk cn's operands load between the products
    const f32x4_t z = {0.f, 0.f, 0.f, 0.f};
    f32x4_t X0 = z, X1 = z, X2 = z, Y0 = z, Y1 = z;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      X0 = mfma(p.whi[ks], shi[ks], X0);
      X1 = mfma(p.whi[ks], slo[ks], X1);
      X2 = mfma(p.wlo[ks], shi[ks], X2);
      if constexpr (EMIT) {
        // the output's Q S0^T on the same B operands (S0 = the state the
        // chunk starts from, in shi / slo until the end of the step)
        Y0 = mfma(po.qa[ks], shi[ks], Y0);
        Y1 = mfma(po.qa[ks], slo[ks], Y1);
      }
    }
    load_w(cn, pn);
    load_rest(cn, pn);
    const f32x4_t U = p.up - (X0 + (X1 + X2));
    ubuf[wave][lane] = U;
    __syncthreads();

    // S_C columns of d_k step `wave`: gamma_C S0 + K^T diag(gamma_C / gamma) U,
    // U over tokens in tau order as the B operand
    if (wave < KS) {
      u32x4_t th[2], tl[2];
#pragma unroll
      for (int kp = 0; kp < 2; ++kp) {
        float x8[8], r8[8];
        cat8(ubuf[2 * kp][lane], ubuf[2 * kp + 1][lane], x8);
        cat8(*reinterpret_cast<const f32x4_t*>(&rbuf[32 * kp + 4 * g]),
             *reinterpret_cast<const f32x4_t*>(&rbuf[32 * kp + 16 + 4 * g]), r8);
#pragma unroll
        for (int j = 0; j < 8; ++j) x8[j] *= r8[j];
        split8(x8, th[kp], tl[kp]);
      }
      f32x4_t acc[2][2];
#pragma unroll
      for (int e = 0; e < 2; ++e) {
        acc[e][0] = sown[e] * p.gC;
        acc[e][1] = z;
#pragma unroll
        for (int kp = 0; kp < 2; ++kp) {
          acc[e][0] = mfma(p.kt[e][kp], th[kp], acc[e][0]);
          acc[e][1] = mfma(p.kt[e][kp], tl[kp], acc[e][1]);
        }
        sown[e] = acc[e][0] + acc[e][1];
      }
      float x8[8];
      cat8(sown[0], sown[1], x8);
      split8(x8, ohi, olo);
      sbuf[wave][0][lane] = ohi;
      sbuf[wave][1][lane] = olo;
    }
    if constexpr (EMIT) {
      // output rows 16w .. of the chunk, this slice's columns (off the
      // state's path, so after the update): diag(gamma) Q S0^T + Aqk U; then
      // the next chunk's output operands load into the same registers
      f32x4_t O0 = z, O1 = z;
      const int nkp = wave < 2 ? 1 : 2;  // token step 1 holds only zeros for rows 0 .. 31
#pragma unroll
      for (int kp = 0; kp < 2; ++kp) {
        if (kp >= nkp) break;
        // U over tokens in tau order: result tiles 2kp and 2kp + 1
        float x8[8];
        cat8(ubuf[2 * kp][lane], ubuf[2 * kp + 1][lane], x8);
        u32x4_t uh, ul;
        split8(x8, uh, ul);
        O0 = mfma(po.ahi[kp], uh, O0);
        O1 = mfma(po.ahi[kp], ul, O1);
        O0 = mfma(po.alo[kp], uh, O0);
      }
      float ov[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) ov[r] = a.q_scale * fmaf(po.gam[r], Y0[r] + Y1[r], O0[r] + O1[r]);
      load_out(min(c + 1, c1 - 1), po);
      // rows past the chunk fall outside the buffer range and are dropped
      // (the first such row is H * d_v floats past the last real one)
      const int n = min(kC, len - c * kC);
      const size_t o0 = (static_cast<size_t>(tok0 + c * kC) * a.H + h) * DV;
      const __amdgpu_buffer_rsrc_t orsrc =
          __builtin_amdgcn_make_buffer_rsrc(a.o + o0, 0, static_cast<int>(((n - 1) * a.H + 1) * DV * 4), 0x00020000);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int t = 16 * wave + 4 * g + r;
        __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(ov[r]), orsrc, (t * a.H * DV + 16 * vs + r16) * 4, 0, 0);
      }
    }
    __syncthreads();
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      shi[ks] = sbuf[ks][0][lane];
      slo[ks] = sbuf[ks][1][lane];
    }
  };

  // chunk c + 2's operands load while chunk c computes (three register
  // sets; past the end the last chunk reloads itself, so that no load sits
  // under a branch).  The pass that emits the output holds the output's
  // operands too and loads one chunk ahead (two sets): three would not fit
  // the registers of two waves per SIMD.
  if constexpr (EMIT) {
    Ops pa, pb;
    if (c1 > c0) {
      load_w(c0, pa);
      load_rest(c0, pa);
      load_out(c0, po);
    }
    for (int c = c0; c < c1; c += 2) {
      step(c, pa, min(c + 1, c1 - 1), pb);
      if (c + 1 >= c1) break;
      step(c + 1, pb, min(c + 2, c1 - 1), pa);
    }
  } else {
    Ops pa, pb, pc;
    if (c1 > c0) {
      load_w(c0, pa);
      load_rest(c0, pa);
      load_w(min(c0 + 1, c1 - 1), pb);
      load_rest(min(c0 + 1, c1 - 1), pb);
    }
    for (int c = c0; c < c1; c += 3) {
      step(c, pa, min(c + 2, c1 - 1), pc);
      if (c + 1 >= c1) break;
      step(c + 1, pb, min(c + 3, c1 - 1), pa);
      if (c + 2 >= c1) break;
      step(c + 2, pc, min(c + 4, c1 - 1), pb);
    }
  }

  // end state: the output slot (one pass, and the last segment of phase 3),
  // or the segment's SE / PI rows (phase 1)
  if (wave < KS && !(a.phase == 3 && seg != a.n_segs - 1)) {
    float* dst = a.phase == 1 ? segb + (pi_rows ? G::PI + static_cast<size_t>(16 * (vs - VT) + r16) * DK
                                                : G::SE + static_cast<size_t>(16 * vs + r16) * DK) +
                                    32 * wave + 4 * g
                              : a.pool + static_cast<size_t>(out) * slot_elems + row_off + 32 * wave + 4 * g;
    *reinterpret_cast<f32x4_t*>(dst) = sown[0];
    *reinterpret_cast<f32x4_t*>(dst + 16) = sown[1];
  }
}

// Segmented scan, phase 2: the start state of every segment,
//   SS(0) = S_in,  SS(1) = SE(0),  SS(g + 1) = SS(g) PI(g) + SE(g),
// in fp32 for state rows 16 vs .. +15 of one (sequence, head).  PI(g)
// passes through LDS; the next segment's PI and SE are loaded into
// registers while this segment's products run.  Thread t owns row t / 16
// and d_k / 16 columns.
template <int DK, int DV>
__global__ __launch_bounds__(256) void gdn_prefill_link_kernel(PrefillArgs a) {
  using G = SegL<DK, DV>;
  constexpr int NCOL = DK / 16;            // columns per thread
  constexpr int NV4 = DK * DK / 4 / 256;   // float4 of PI per thread
  const int vs = blockIdx.x, h = blockIdx.y, s = blockIdx.z;
  const int tok0 = a.cu[s], len = a.cu[s + 1] - tok0;
  const int in = a.in_idx[s], out = a.out_idx[s];
  if (tok0 < 0 || len < 0 || len > a.max_len) return;                       // the scan reports it
  if (in < -1 || in >= a.n_slots || out < 0 || out >= a.n_slots) return;
  __shared__ __align__(16) float pis[DK * DK];
  __shared__ float srow[16][DK + 1];
  const int t = threadIdx.x, r = t / 16, col0 = (t % 16) * NCOL;
  const size_t seg_stride = static_cast<size_t>(a.H) * G::TOTAL;  // between segments of one (s, h)
  float* base = a.seg + (static_cast<size_t>(s) * a.n_segs * a.H + h) * G::TOTAL;
  const size_t row = static_cast<size_t>(16 * vs + r) * DK;
  f32x4_t pre[NV4];
  float se[NCOL];
  auto fetch = [&](int g) {
    const float* sg = base + g * seg_stride;
#pragma unroll
    for (int i = 0; i < NV4; ++i) pre[i] = reinterpret_cast<const f32x4_t*>(sg + G::PI)[t + 256 * i];
#pragma unroll
    for (int j = 0; j < NCOL; ++j) se[j] = sg[G::SE + row + col0 + j];
  };
  float acc[NCOL];
  {
    const float* src = a.pool + (static_cast<size_t>(max(in, 0)) * a.H + h) * DV * DK + row + col0;
#pragma unroll
    for (int j = 0; j < NCOL; ++j) acc[j] = in >= 0 ? src[j] : 0.f;
  }
  // SS(0): the input state; SS(1): the first segment's end state, which
  // phase 1 computed from the input state
#pragma unroll
  for (int j = 0; j < NCOL; ++j) base[G::SS + row + col0 + j] = acc[j];
#pragma unroll
  for (int j = 0; j < NCOL; ++j) acc[j] = base[G::SE + row + col0 + j];
  fetch(min(1, a.n_segs - 1));
  for (int g = 1;; ++g) {
    float* sg = base + g * seg_stride;
#pragma unroll
    for (int j = 0; j < NCOL; ++j) {
      sg[G::SS + row + col0 + j] = acc[j];
      srow[r][col0 + j] = acc[j];
    }
    if (g + 1 >= a.n_segs) break;
#pragma unroll
    for (int i = 0; i < NV4; ++i) reinterpret_cast<f32x4_t*>(pis)[t + 256 * i] = pre[i];
#pragma unroll
    for (int j = 0; j < NCOL; ++j) acc[j] = se[j];
    __syncthreads();
    fetch(min(g + 1, a.n_segs - 1));  // (the last round reloads a segment that exists)
    for (int k = 0; k < DK; ++k) {
      const float x = srow[r][k];
#pragma unroll
      for (int j = 0; j < NCOL; ++j) acc[j] = fmaf(x, pis[k * DK + col0 + j], acc[j]);
    }
    __syncthreads();
  }
}

size_t block_bytes(int dk, int dv) {
  if (dk == 128) return 16 * static_cast<size_t>(dv == 128 ? PL<128, 128>::TOTAL : PL<128, 64>::TOTAL);
  return 16 * static_cast<size_t>(dv == 128 ? PL<64, 128>::TOTAL : PL<64, 64>::TOTAL);
}

int check(const had_gdn_prefill_desc* d) {
  if (!d) return fail(HAD_ERR_INVALID_ARG, "gdn_prefill: desc is NULL");
  if (d->n_seqs < 1 || d->H < 1 || d->n_slots < 1 || d->max_len < 0)
    return fail(HAD_ERR_INVALID_ARG, "gdn_prefill: bad counts (n_seqs=%d H=%d n_slots=%d max_len=%d)", d->n_seqs,
                d->H, d->n_slots, d->max_len);
  if ((d->d_k != 64 && d->d_k != 128) || (d->d_v != 64 && d->d_v != 128))
    return fail(HAD_ERR_UNSUPPORTED_SHAPE, "gdn_prefill: d_k=%d d_v=%d (supported: 64, 128)", d->d_k, d->d_v);
  if (d->flags & ~HAD_GDN_RAW_GATES) return fail(HAD_ERR_INVALID_ARG, "gdn_prefill: unknown flags 0x%x", d->flags);
  if (d->n_segments < 0) return fail(HAD_ERR_INVALID_ARG, "gdn_prefill: n_segments %d < 0", d->n_segments);
  return HAD_OK;
}

// Segments of the scan.  One pass keeps n_seqs x H x d_v/16 workgroups busy
// along a chain of every chunk; segments run side by side at the price of a
// second scan pass (twice the rows: the transition) and the link, and the
// chain becomes two segment lengths (so two segments gain nothing).  Worth
// it for long prompts that leave most CUs idle: segments of >= 32 chunks,
// at most 512 phase-3 workgroups (two per CU), at least three segments.
int plan_segments(const had_gdn_prefill_desc* d) {
  const int chunks = (d->max_len + kC - 1) / kC;
  int g;
  if (d->n_segments > 0) {
    g = d->n_segments;
  } else {
    const int per_seg = d->n_seqs * d->H * (d->d_v / 16);
    g = std::min(chunks / 32, 512 / std::max(per_seg, 1));
    if (g < 3) g = 1;
  }
  return std::max(1, std::min(g, std::max(chunks, 1)));
}

size_t chunk_bytes(const had_gdn_prefill_desc* d) {
  const size_t chunks = static_cast<size_t>((d->max_len + kC - 1) / kC);
  return (static_cast<size_t>(d->n_seqs) * chunks * d->H * block_bytes(d->d_k, d->d_v) + 255) & ~size_t(255);
}

size_t seg_bytes(const had_gdn_prefill_desc* d) {
  const int g = plan_segments(d);
  if (g < 2) return 0;
  const size_t per = static_cast<size_t>(d->d_k) * d->d_k + 2 * static_cast<size_t>(d->d_v) * d->d_k;
  return static_cast<size_t>(d->n_seqs) * g * d->H * per * sizeof(float);
}

template <int DK, int DV>
int launch(const had_gdn_prefill_desc* d, PrefillArgs a, hipStream_t st) {
  if (a.max_chunks > 0) {
    hipLaunchKernelGGL((gdn_prefill_prep_kernel<DK, DV>), dim3(a.max_chunks, d->H, d->n_seqs), dim3(256), 0, st, a);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return fail(HAD_ERR_HIP, "gdn_prefill: prep launch: %s", hipGetErrorString(e));
  }
  const int items = d->n_seqs * d->H * a.n_segs;
  hipError_t e;
  if (a.n_segs > 1) {
    a.phase = 1;
    const int items1 = d->n_seqs * d->H * (a.n_segs - 1);  // every segment but the last
    hipLaunchKernelGGL((gdn_prefill_scan_kernel<DK, DV, false>), dim3((items1 + 7) / 8 * 8 * (DV / 16 + DK / 16)),
                       dim3(256), 0, st, a);
    e = hipGetLastError();
    if (e != hipSuccess) return fail(HAD_ERR_HIP, "gdn_prefill: segment scan launch: %s", hipGetErrorString(e));
    hipLaunchKernelGGL((gdn_prefill_link_kernel<DK, DV>), dim3(DV / 16, d->H, d->n_seqs), dim3(256), 0, st, a);
    e = hipGetLastError();
    if (e != hipSuccess) return fail(HAD_ERR_HIP, "gdn_prefill: link launch: %s", hipGetErrorString(e));
    a.phase = 3;
  } else {
    a.phase = 0;
  }
  hipLaunchKernelGGL((gdn_prefill_scan_kernel<DK, DV, true>), dim3((items + 7) / 8 * 8 * (DV / 16)), dim3(256), 0, st,
                     a);
  e = hipGetLastError();
  if (e != hipSuccess) return fail(HAD_ERR_HIP, "gdn_prefill: scan launch: %s", hipGetErrorString(e));
  return HAD_OK;
}

}  // namespace
}  // namespace had

extern "C" {

size_t had_gdn_prefill_workspace_bytes(const had_gdn_prefill_desc* d) {
  if (had::check(d) != HAD_OK) return 0;
  return had::chunk_bytes(d) + had::seg_bytes(d);
}

int had_gdn_prefill(const had_gdn_prefill_desc* d, const had_gdn_prefill_ptrs* p, void* stream) {
  int st = had::check(d);
  if (st != HAD_OK) return st;
  if (!p || !p->state_pool || !p->in_idx || !p->out_idx || !p->cu_seqlens || !p->q || !p->k || !p->v || !p->alpha ||
      !p->beta || !p->o)
    return fail(HAD_ERR_INVALID_ARG, "gdn_prefill: NULL pointer in ptrs");
  const size_t need = had_gdn_prefill_workspace_bytes(d);
  if (need > 0 && (!p->workspace || p->workspace_bytes < need))
    return fail(HAD_ERR_WORKSPACE_TOO_SMALL, "gdn_prefill: workspace %zu bytes, need %zu", p->workspace_bytes, need);
  if ((reinterpret_cast<uintptr_t>(p->workspace) | reinterpret_cast<uintptr_t>(p->state_pool) |
       reinterpret_cast<uintptr_t>(p->q) | reinterpret_cast<uintptr_t>(p->k) | reinterpret_cast<uintptr_t>(p->v)) &
      15u)
    return fail(HAD_ERR_INVALID_ARG, "gdn_prefill: workspace, state_pool, q, k and v must be 16-byte aligned");
  had::PrefillArgs a{};
  a.pool = p->state_pool;
  a.in_idx = p->in_idx;
  a.out_idx = p->out_idx;
  a.cu = p->cu_seqlens;
  a.q = static_cast<const uint16_t*>(p->q);
  a.k = static_cast<const uint16_t*>(p->k);
  a.v = static_cast<const uint16_t*>(p->v);
  a.alpha = p->alpha;
  a.beta = p->beta;
  a.o = p->o;
  a.ws = static_cast<had::u32x4_t*>(p->workspace);
  a.d_err = p->d_err;
  a.n_seqs = d->n_seqs;
  a.H = d->H;
  a.n_slots = d->n_slots;
  a.max_len = d->max_len;
  a.max_chunks = (d->max_len + had::kC - 1) / had::kC;
  a.raw_gates = (d->flags & HAD_GDN_RAW_GATES) ? 1 : 0;
  a.q_scale = d->q_scale;
  a.n_segs = had::plan_segments(d);
  a.seg_chunks = (a.max_chunks + a.n_segs - 1) / a.n_segs;
  a.seg = a.n_segs > 1 ? reinterpret_cast<float*>(static_cast<char*>(p->workspace) + had::chunk_bytes(d)) : nullptr;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (d->d_k == 128 && d->d_v == 128) st = had::launch<128, 128>(d, a, s);
  else if (d->d_k == 128) st = had::launch<128, 64>(d, a, s);
  else if (d->d_v == 128) st = had::launch<64, 128>(d, a, s);
  else st = had::launch<64, 64>(d, a, s);
  return st == HAD_OK ? had::ok() : st;
}

}  // extern "C"
