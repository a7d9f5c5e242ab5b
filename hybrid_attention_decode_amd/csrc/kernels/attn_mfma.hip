// Split-K GQA decode attention, MFMA path (16 or more query rows per KV
// head, e.g. GQA group 16 x 4 draft tokens when a speculative draft is
// verified: zubnet.ai TokenSpeed article, second paragraph, speculative
// decoding; 24-ai.news long-context table for the context range).
//
// Same operation and partial format as the VALU path: for the rows of one
// (sequence, KV head), softmax(sm_scale q K^T) V over the split's tokens,
// causal inside the draft, written as unnormalised (o, m, l) in base 2.
//
// gfx950 mapping (one workgroup = 4 waves, wave w owns query rows
// 16w .. 16w+15 of the launch; tiles of 32 tokens):
//  * K and V tiles are staged once per workgroup: global -> registers
//    (prefetched one tile ahead) -> LDS, double-buffered.  K keeps its
//    row-major layout with the 16-byte chunks XOR-swizzled by token (so 16
//    lanes reading 16 tokens hit 16 different bank groups); V is written
//    d-major (transposed) for the PV operand.
//  * S^T = K Q^T with v_mfma_f32_16x16x32_bf16 (A = K rows, B = q rows held
//    in registers): the C layout leaves each lane 8 token scores of ONE query
//    row, which is exactly the B operand P^T of O^T = V^T P^T once the 32
//    tokens are taken in the order tau(g, i) = 4g + i (i < 4), 16 + 4g + i-4
//    (i >= 4) -- so P never goes through LDS, and the online-softmax
//    rescale of a lane's O^T accumulators uses the lane's own row state.
//  * Row maxima and sums combine the 4 lanes of a row with two bpermutes.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "attn_internal.h"
#include "kcommon.h"

namespace had {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

constexpr int kMWaves = 4;
constexpr int kMRows = 16 * kMWaves;  // query rows per launch
constexpr int kMTT = 32;              // tokens per tile

template <int D>
struct MCfg {
  static constexpr int KS = D / 32;              // QK k-steps (32 d each)
  static constexpr int MB = D / 16;              // PV output blocks (16 d each)
  static constexpr int CPR = D / 8;              // 16-byte chunks per K/V row
  static constexpr int CPT = kMTT * CPR / 256;   // chunks per thread per tile (K, and again V)
  static constexpr int SWZ = (CPR < 16 ? CPR : 16) - 1;
  static constexpr int VTP = kMTT + 4;           // bf16 per d-row of the transposed V tile (padded)
  static_assert(CPT >= 1, "unsupported head_dim");
};

template <int D>
struct MLds {
  uint4 k[2][kMTT * MCfg<D>::CPR];
  uint16_t vt[2][D * MCfg<D>::VTP];
  int32_t pages[kMaxPagesPerSplit];
  int err;
};

__device__ __forceinline__ bf16x8_t as_bf16x8(uint4 v) { return __builtin_bit_cast(bf16x8_t, v); }

template <int D>
__global__ __launch_bounds__(256, 2) void attn_mfma_kernel(ValuArgs a) {
  using C = MCfg<D>;
  __shared__ MLds<D> sh;
  const int sp = blockIdx.x, h = blockIdx.y, s = blockIdx.z;
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int r16 = lane & 15, g = lane >> 4;
  const int P = a.page_size;

  const int pg0 = static_cast<int>(static_cast<int64_t>(sp) * a.n_pages_plan / a.num_splits);
  const int pg1_plan = static_cast<int>(static_cast<int64_t>(sp + 1) * a.n_pages_plan / a.num_splits);
  const int npg_plan = pg1_plan - pg0;
  const int32_t* pt_row = a.page_table + static_cast<size_t>(s) * a.max_pages;
  const int L = a.seq_lens[s];
  const bool bad_len = L < a.q_len || L > a.max_pages * P;
  const int n_pages = bad_len ? 0 : (L + P - 1) / P;
  const int npg = max(min(pg1_plan, n_pages) - pg0, 0);
  const int tok0 = pg0 * P;
  const int tok_end = npg > 0 ? min((pg0 + npg) * P, L) : tok0;  // this split's tokens: [tok0, tok_end)
  const int n_tiles = (tok_end - tok0 + kMTT - 1) / kMTT;

  int errs = (bad_len && tid == 0) ? HAD_DERR_SEQLEN : 0;
  if (tid == 0) sh.err = 0;
  for (int i = tid; i < npg_plan; i += blockDim.x) {
    const int pid = pt_row[pg0 + i];
    const bool ok = pid >= 0 && pid < a.num_pages;
    if (!ok && i < npg) errs |= HAD_DERR_PAGE;
    sh.pages[i] = ok ? pid : -1;
  }

  // q rows of this wave as the B operand of S^T = K Q^T: lane (r16, g) holds
  // row 16*wave + r16, dims 32*ks + 8g .. +8 (zero for padding rows)
  const int row = a.row_base + 16 * wave + r16;
  const bool row_ok = row < a.rows;
  uint4 qb[C::KS];
  {
    const int rc = row_ok ? row : 0;
    const uint16_t* qp = a.q + ((static_cast<size_t>(s) * a.q_len + rc / a.G) * a.H_q + h * a.G + rc % a.G) * D;
#pragma unroll
    for (int ks = 0; ks < C::KS; ++ks) {
      const uint4 v = *reinterpret_cast<const uint4*>(qp + 32 * ks + 8 * g);
      qb[ks] = row_ok ? v : make_uint4(0u, 0u, 0u, 0u);
    }
  }
  const int lim = row_ok ? (L - a.q_len + row / a.G + 1) : L;  // visible keys of this lane's row

  __syncthreads();

  // ---- K/V staging: thread tid moves chunks id = tid + 256*i of the tile
  uint4 kreg[C::CPT], vreg[C::CPT];
  auto load_regs = [&](int tile) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < C::CPT; ++i) {
      const int id = tid + 256 * i;
      const int tt = id / C::CPR, c = id % C::CPR;
      const int tok = min(tok0 + tile * kMTT + tt, max(tok_end - 1, tok0));
      int pid = sh.pages[min(tok / P - pg0, max(npg - 1, 0))];
      pid = pid < 0 ? 0 : pid;
      const size_t off = ((static_cast<size_t>(pid) * a.H_kv + h) * P + tok % P) * D + c * 8;
      kreg[i] = *reinterpret_cast<const uint4*>(a.k_pool + off);
      vreg[i] = *reinterpret_cast<const uint4*>(a.v_pool + off);
    }
  };
  auto store_lds = [&](int tile, int b) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < C::CPT; ++i) {
      const int id = tid + 256 * i;
      const int tt = id / C::CPR, c = id % C::CPR;
      const int tok = tok0 + tile * kMTT + tt;
      const bool tok_ok = tok < tok_end && sh.pages[min(tok / P - pg0, max(npg - 1, 0))] >= 0;
      sh.k[b][tt * C::CPR + (c ^ (tt & C::SWZ))] = kreg[i];
      // V transposed; rows that must not count (past the split, past the
      // length, unchecked page) are written as zeros so stale bits never meet
      // a zero probability
      const uint4 v = tok_ok ? vreg[i] : make_uint4(0u, 0u, 0u, 0u);
      const uint32_t w[4] = {v.x, v.y, v.z, v.w};
      uint16_t* vt = &sh.vt[b][(8 * c) * C::VTP + tt];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        vt[(2 * e) * C::VTP] = static_cast<uint16_t>(w[e] & 0xffffu);
        vt[(2 * e + 1) * C::VTP] = static_cast<uint16_t>(w[e] >> 16);
      }
    }
  };

  f32x4_t o[C::MB];
#pragma unroll
  for (int mb = 0; mb < C::MB; ++mb) o[mb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY, l_run = 0.f;

  if (n_tiles > 0) load_regs(0);
  for (int tile = 0; tile < n_tiles; ++tile) {
    const int b = tile & 1;
    store_lds(tile, b);
    if (tile + 1 < n_tiles) load_regs(tile + 1);
    __syncthreads();

    // ---- S^T for the 32 tokens: two 16-token blocks, KS k-steps each
    float sc[8];
#pragma unroll
    for (int tb = 0; tb < 2; ++tb) {
      f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
      const int tt = 16 * tb + r16;  // A-operand row = token
#pragma unroll
      for (int ks = 0; ks < C::KS; ++ks) {
        const int c = 4 * ks + g;
        const uint4 kv = sh.k[b][tt * C::CPR + (c ^ (tt & C::SWZ))];
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(kv), as_bf16x8(qb[ks]), acc, 0, 0, 0);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) sc[4 * tb + i] = acc[i] * a.scale_log2;
    }
    // tokens of slot i: tau(g, i) = 4g + i and 16 + 4g + i
    const int pos0 = tok0 + tile * kMTT;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int pos = pos0 + (i < 4 ? 4 * g + i : 16 + 4 * g + (i - 4));
      if (pos >= tok_end || pos >= lim) sc[i] = -INFINITY;
    }

    // ---- online softmax for this lane's row (4 lanes per row: g = 0..3)
    float mt = sc[0];
#pragma unroll
    for (int i = 1; i < 8; ++i) mt = fmaxf(mt, sc[i]);
    mt = fmaxf(mt, shfl_xor_f(mt, 16));
    mt = fmaxf(mt, shfl_xor_f(mt, 32));
    const float m_new = fmaxf(m_run, mt);
    const float m_sub = (m_new == -INFINITY) ? 0.f : m_new;
    const float alpha = exp2f(m_run - m_sub);
    uint32_t pw[4];
    float lsum = 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      pw[i] = pack_bf16x2(exp2f(sc[2 * i] - m_sub), exp2f(sc[2 * i + 1] - m_sub));
      lsum += bf16_lo(pw[i]) + bf16_hi(pw[i]);
    }
    l_run = l_run * alpha + lsum;
    m_run = m_new;
    const uint4 pb = make_uint4(pw[0], pw[1], pw[2], pw[3]);

    // ---- O^T += V^T P^T over the 32 tokens, one MFMA per 16 output dims
#pragma unroll
    for (int mb = 0; mb < C::MB; ++mb) {
      const uint16_t* vrow = &sh.vt[b][(16 * mb + r16) * C::VTP];
      const uint2 lo = *reinterpret_cast<const uint2*>(vrow + 4 * g);
      const uint2 hi = *reinterpret_cast<const uint2*>(vrow + 16 + 4 * g);
      const uint4 va = make_uint4(lo.x, lo.y, hi.x, hi.y);
      o[mb] = o[mb] * alpha;
      o[mb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(va), as_bf16x8(pb), o[mb], 0, 0, 0);
    }
  }

  // ---- row totals and the partial store (no cross-wave merge: waves own rows)
  l_run += shfl_xor_f(l_run, 16);
  l_run += shfl_xor_f(l_run, 32);
  if (errs) atomicOr(&sh.err, errs);
  __syncthreads();
  if (tid == 0 && sh.err) set_err(a.d_err, sh.err);
  if (row_ok) {
    const size_t unit = (static_cast<size_t>(s) * a.H_kv + h) * a.num_splits + sp;
    float* op = a.ws_o + (unit * a.rows + row) * D;
#pragma unroll
    for (int mb = 0; mb < C::MB; ++mb)
      *reinterpret_cast<float4*>(op + 16 * mb + 4 * g) = make_float4(o[mb][0], o[mb][1], o[mb][2], o[mb][3]);
    if (g == 0) {
      a.ws_ml[(unit * a.rows + row) * 2 + 0] = m_run;
      a.ws_ml[(unit * a.rows + row) * 2 + 1] = l_run;
    }
  }
}

}  // namespace

hipError_t launch_attn_mfma(const ValuArgs& a_in, int head_dim, dim3 grid, hipStream_t stream) {
  ValuArgs a = a_in;
  hipError_t e = hipSuccess;
  for (int rb = 0; rb < a.rows && e == hipSuccess; rb += kMRows) {
    a.row_base = rb;
    switch (head_dim) {
      case 64: hipLaunchKernelGGL(attn_mfma_kernel<64>, grid, dim3(256), 0, stream, a); break;
      case 128: hipLaunchKernelGGL(attn_mfma_kernel<128>, grid, dim3(256), 0, stream, a); break;
      case 256: hipLaunchKernelGGL(attn_mfma_kernel<256>, grid, dim3(256), 0, stream, a); break;
      default: return hipErrorInvalidValue;
    }
    e = hipGetLastError();
  }
  return e;
}

}  // namespace had
