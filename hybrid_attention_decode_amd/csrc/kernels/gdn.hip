// Gated delta rule update of slot-addressed recurrent states.
//
// For sequence s, head h, with S (d_v x d_k, fp32) read from slot in_idx[s]
// (zero state for -1), for each of the T tokens:
//   S <- alpha S (I - beta k k^T) + beta v k^T     evaluated as
//   u = beta (v - alpha S k),  S <- alpha S + u k^T
//   o = q_scale * S q,  and S is stored to slot out_idx[s][t].
// Gated DeltaNet layers of the hybrid model (24-ai.news TokenSpeed article,
// model paragraph; recurrence of Yang, Kautz & Hatamizadeh, ICLR 2025).  The
// state never moves between slots by copy: a step reads one slot index and
// writes another (zubnet.ai TokenSpeed article, second paragraph,
// current_input_indices; 24-ai.news "Mamba State Update", O(1) pointer
// update).  With T > 1 the state stays in registers across tokens and every
// token's state is written as a checkpoint; all tokens' inputs are loaded
// before the first is processed.
//
// Mapping: one wave per (s, h, block of RPW = 4 rows of S), so the 128 rows
// of 8 heads of 128 x 128 take 256 waves, one per CU, each its own
// workgroup; a grid of 1024 waves or more (a batch of sequences) puts four
// waves in a workgroup, a quarter of the workgroups to dispatch (16
// sequences x 8 heads: 5.9 instead of 6.2 us per layer; two waves per
// workgroup 6.1, eight 5.9).  Lane (r, c) holds row
// r's columns {4c + 64i .. 4c + 64i + 3} (16 lanes per row), so each row's
// lanes read a contiguous 256-byte segment per float4; the dot products S k
// and S q are all-reduced across those 16 lanes with four DPP adds.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../host/status.h"
#include "had.h"
#include "kcommon.h"

using had::fail;

namespace had {
namespace {

struct GdnArgs {
  float* pool;
  const int32_t* in_idx;
  const int32_t* out_idx;
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  const float* alpha;
  const float* beta;
  float* o;
  int32_t* d_err;
  int T, H, d_v, n_slots;
  float q_scale;
  int raw_gates;  // alpha / beta hold g and b: alpha = exp(g), beta = sigmoid(b)
};

constexpr int kRPW = 4;          // state rows per wave
constexpr int kLPR = 64 / kRPW;  // lanes per row

// sum over the kLPR lanes of a row (groups of 8, then the two halves of a
// 16-lane row)
__device__ __forceinline__ float sum_row(float x) {
  x += dpp<DPP_QUAD_XOR1>(x);
  x += dpp<DPP_QUAD_XOR2>(x);
  x += dpp<DPP_ROW_HALF_MIRROR>(x);
  if constexpr (kLPR == 16) x += dpp<DPP_ROW_ROR8>(x);
  return x;
}

// TM: compile-time bound on T.  Every token's inputs (q, k, v row, gates,
// out slot) are loaded before the first token is processed -- tokens past T
// reload the last one, so no load sits under a branch -- and the recurrence
// then runs from registers; only the state store of each token waits on
// the previous token.
template <int DK, int TM, int WPB>
__global__ __launch_bounds__(64 * WPB) void gdn_kernel(GdnArgs a) {
  static_assert(kLPR == 8 || kLPR == 16, "row sums over 8 or 16 lanes");
  constexpr int NC = DK / (4 * kLPR);  // float4 column chunks per lane
  constexpr int CS = 4 * kLPR;         // columns between a lane's chunks
  const int rb = blockIdx.x * WPB + (threadIdx.x >> 6), h = blockIdx.y, s = blockIdx.z;  // row block
  const int lane = threadIdx.x & 63;
  const int r = lane / kLPR, c = lane % kLPR;
  const int row = rb * kRPW + r;
  const size_t head_elems = static_cast<size_t>(a.d_v) * DK;
  const size_t row_off = static_cast<size_t>(h) * head_elems + static_cast<size_t>(row) * DK;
  const size_t slot_elems = static_cast<size_t>(a.H) * head_elems;

  // token inputs first (independent of the state)
  uint2 kw[TM][NC], qw[TM][NC];
  float vi[TM], al[TM], be[TM];
  int outs[TM];
#pragma unroll
  for (int t = 0; t < TM; ++t) {
    const int tt = min(t, a.T - 1);
    const size_t th = (static_cast<size_t>(s) * a.T + tt) * a.H + h;
    const uint16_t* kp = a.k + th * DK;
    const uint16_t* qp = a.q + th * DK;
#pragma unroll
    for (int i = 0; i < NC; ++i) {
      kw[t][i] = *reinterpret_cast<const uint2*>(kp + 4 * c + CS * i);
      qw[t][i] = *reinterpret_cast<const uint2*>(qp + 4 * c + CS * i);
    }
    vi[t] = bf16_to_f32(a.v[th * a.d_v + row]);
    al[t] = a.alpha[th];
    be[t] = a.beta[th];
    outs[t] = a.out_idx[static_cast<size_t>(s) * a.T + tt];
  }

  int in = a.in_idx[s];
  if (in < -1 || in >= a.n_slots) {
    if (lane == 0) set_err(a.d_err, HAD_DERR_SLOT);
    in = -1;
  }
  float S[NC][4];
  {
    // a clamped, unconditional load; the zero state (in = -1) is selected
    // after it.  At T = 1 with the non-temporal hint: the state is read once
    // per step, and left out of the caches it leaves them to the rest of the
    // step (agentic loop 2961 -> 3012, 16-sequence batch 1323 -> 1392
    // steps/s; at T = 4 the hint costs 0.15 us per layer and is not used)
    const float* src = a.pool + static_cast<size_t>(max(in, 0)) * slot_elems + row_off;
    typedef float f32x4_t __attribute__((ext_vector_type(4)));
#pragma unroll
    for (int i = 0; i < NC; ++i) {
      const f32x4_t* sp = reinterpret_cast<const f32x4_t*>(src + 4 * c + CS * i);
      const f32x4_t t4 = TM == 1 ? __builtin_nontemporal_load(sp) : *sp;
      S[i][0] = in >= 0 ? t4.x : 0.f;
      S[i][1] = in >= 0 ? t4.y : 0.f;
      S[i][2] = in >= 0 ? t4.z : 0.f;
      S[i][3] = in >= 0 ? t4.w : 0.f;
    }
  }

#pragma unroll
  for (int t = 0; t < TM; ++t) {
    if (t >= a.T) break;
    const size_t th = (static_cast<size_t>(s) * a.T + t) * a.H + h;
    float alt = al[t], bet = be[t];
    if (a.raw_gates) {
      alt = expf(alt);
      bet = 1.f / (1.f + expf(-bet));
    }
    float kk[NC][4], qq[NC][4];
#pragma unroll
    for (int i = 0; i < NC; ++i) {
      kk[i][0] = bf16_lo(kw[t][i].x); kk[i][1] = bf16_hi(kw[t][i].x); kk[i][2] = bf16_lo(kw[t][i].y); kk[i][3] = bf16_hi(kw[t][i].y);
      qq[i][0] = bf16_lo(qw[t][i].x); qq[i][1] = bf16_hi(qw[t][i].x); qq[i][2] = bf16_lo(qw[t][i].y); qq[i][3] = bf16_hi(qw[t][i].y);
    }
    float sk = 0.f;
#pragma unroll
    for (int i = 0; i < NC; ++i)
#pragma unroll
      for (int e = 0; e < 4; ++e) sk = fmaf(S[i][e], kk[i][e], sk);
    sk = sum_row(sk);
    const float u = bet * (vi[t] - alt * sk);
    float sq = 0.f;
#pragma unroll
    for (int i = 0; i < NC; ++i)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        S[i][e] = fmaf(u, kk[i][e], alt * S[i][e]);
        sq = fmaf(S[i][e], qq[i][e], sq);
      }
    sq = sum_row(sq);
    if (c == 0) a.o[th * a.d_v + row] = a.q_scale * sq;
    const int out = outs[t];
    if (out < 0 || out >= a.n_slots) {
      if (lane == 0) set_err(a.d_err, HAD_DERR_SLOT);
      continue;
    }
    float* dst = a.pool + static_cast<size_t>(out) * slot_elems + row_off;
#pragma unroll
    for (int i = 0; i < NC; ++i)
      *reinterpret_cast<float4*>(dst + 4 * c + CS * i) = make_float4(S[i][0], S[i][1], S[i][2], S[i][3]);
  }
}

}  // namespace
}  // namespace had

extern "C" int had_gdn_state_update(const had_gdn_desc* d, const had_gdn_ptrs* p, void* stream) {
  if (!d || !p) return fail(HAD_ERR_INVALID_ARG, "gdn_state_update: NULL argument");
  if (d->n_seqs < 0 || d->H < 1 || d->n_slots < 1 || d->T < 1 || d->T > 8)
    return fail(HAD_ERR_INVALID_ARG, "gdn_state_update: bad sizes (n_seqs=%d T=%d H=%d n_slots=%d)", d->n_seqs, d->T,
                d->H, d->n_slots);
  if ((d->d_k != 64 && d->d_k != 128) || (d->d_v != 64 && d->d_v != 128))
    return fail(HAD_ERR_UNSUPPORTED_SHAPE, "gdn_state_update: d_k=%d d_v=%d must be 64 or 128", d->d_k, d->d_v);
  if (d->flags & ~HAD_GDN_RAW_GATES) return fail(HAD_ERR_INVALID_ARG, "gdn_state_update: unknown flags 0x%x", d->flags);
  if (!p->state_pool || !p->in_idx || !p->out_idx || !p->q || !p->k || !p->v || !p->alpha || !p->beta || !p->o)
    return fail(HAD_ERR_INVALID_ARG, "gdn_state_update: NULL pointer in ptrs");
  if ((reinterpret_cast<uintptr_t>(p->state_pool) & 15u) != 0 || (reinterpret_cast<uintptr_t>(p->q) & 7u) != 0 ||
      (reinterpret_cast<uintptr_t>(p->k) & 7u) != 0)
    return fail(HAD_ERR_INVALID_ARG, "gdn_state_update: state_pool must be 16-byte and q, k 8-byte aligned");
  if (d->n_seqs == 0) return had::ok();
  had::GdnArgs a{};
  a.pool = p->state_pool;
  a.in_idx = p->in_idx;
  a.out_idx = p->out_idx;
  a.q = static_cast<const uint16_t*>(p->q);
  a.k = static_cast<const uint16_t*>(p->k);
  a.v = static_cast<const uint16_t*>(p->v);
  a.alpha = p->alpha;
  a.beta = p->beta;
  a.o = p->o;
  a.d_err = p->d_err;
  a.T = d->T;
  a.raw_gates = (d->flags & HAD_GDN_RAW_GATES) ? 1 : 0;
  a.H = d->H;
  a.d_v = d->d_v;
  a.n_slots = d->n_slots;
  a.q_scale = d->q_scale;
  // waves per workgroup: 4 for grids of 1024 waves or more (d_v / kRPW row
  // blocks per head, 16 or 32, divide by 4), else 1
  const bool grouped = static_cast<int64_t>(d->n_seqs) * d->H * (d->d_v / had::kRPW) >= 1024;
  const dim3 grid(d->d_v / had::kRPW / (grouped ? 4 : 1), d->H, d->n_seqs);
  hipStream_t s = static_cast<hipStream_t>(stream);
  // the token bound the kernel is compiled for: 1, 4 or 8
  const int tm = d->T == 1 ? 1 : d->T <= 4 ? 4 : 8;
  switch ((d->d_k == 64 ? 0 : 16) + tm * 2 + (grouped ? 1 : 0)) {
    case 2: hipLaunchKernelGGL((had::gdn_kernel<64, 1, 1>), grid, dim3(64), 0, s, a); break;
    case 3: hipLaunchKernelGGL((had::gdn_kernel<64, 1, 4>), grid, dim3(256), 0, s, a); break;
    case 8: hipLaunchKernelGGL((had::gdn_kernel<64, 4, 1>), grid, dim3(64), 0, s, a); break;
    case 9: hipLaunchKernelGGL((had::gdn_kernel<64, 4, 4>), grid, dim3(256), 0, s, a); break;
    case 16: hipLaunchKernelGGL((had::gdn_kernel<64, 8, 1>), grid, dim3(64), 0, s, a); break;
    case 17: hipLaunchKernelGGL((had::gdn_kernel<64, 8, 4>), grid, dim3(256), 0, s, a); break;
    case 18: hipLaunchKernelGGL((had::gdn_kernel<128, 1, 1>), grid, dim3(64), 0, s, a); break;
    case 19: hipLaunchKernelGGL((had::gdn_kernel<128, 1, 4>), grid, dim3(256), 0, s, a); break;
    case 24: hipLaunchKernelGGL((had::gdn_kernel<128, 4, 1>), grid, dim3(64), 0, s, a); break;
    case 25: hipLaunchKernelGGL((had::gdn_kernel<128, 4, 4>), grid, dim3(256), 0, s, a); break;
    case 32: hipLaunchKernelGGL((had::gdn_kernel<128, 8, 1>), grid, dim3(64), 0, s, a); break;
    default: hipLaunchKernelGGL((had::gdn_kernel<128, 8, 4>), grid, dim3(256), 0, s, a); break;
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(HAD_ERR_HIP, "gdn_state_update: launch: %s", hipGetErrorString(e));
  return had::ok();
}
