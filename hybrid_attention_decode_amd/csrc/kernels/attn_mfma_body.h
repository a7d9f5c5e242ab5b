// Body of the MFMA split-K decode partial (16 or more query rows per KV
// head), shared by its own kernel (attn_mfma.hip) and the one-launch cascade
// (attn_cascade.hip).  The operation and the gfx950 mapping are described in
// attn_mfma.hip.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "attn_internal.h"
#include "kcommon.h"

namespace had {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));  // staging registers (first-class vectors)

constexpr int kMWaves = 8;                 // two teams of four waves
constexpr int kMRows = 64;                 // query rows per launch (16 per wave of a team)
constexpr int kMTeamTok = 32;              // tokens per team per iteration
constexpr int kMTile = 2 * kMTeamTok;      // tokens staged per iteration

template <int D>
struct MCfg {
  static constexpr int KS = D / 32;              // QK k-steps (32 d each)
  static constexpr int MB = D / 16;              // PV output blocks (16 d each)
  static constexpr int CPR = D / 8;              // 16-byte chunks per K/V row
  static constexpr int TPT = CPR / 8;            // consecutive tokens per staging thread (4, 2, 1)
  static constexpr int GPT = kMTeamTok / TPT;    // token groups per team
  static constexpr int CPW = 64 / GPT;           // chunk columns per staging wave
  static constexpr int SWZ = (CPR < 16 ? CPR : 16) - 1;
  static constexpr int VTP = kMTeamTok + 4;      // bf16 pitch of a transposed V row (padded)
  static constexpr int OP = D + 4;               // float pitch of a team-merge row (padded)
  static_assert(CPW * 4 == CPR, "staging map must cover every chunk column");
};

template <int D>
struct MTiles {
  u32x4_t k[2][kMTile * MCfg<D>::CPR];
  uint16_t vt[2][2][D * MCfg<D>::VTP];  // [buffer][team][d][token]
};

template <int D>
struct MMerge {
  float o[4][16][MCfg<D>::OP];
  float ml[4][16][2];
};

template <int D>
struct MLds {
  union {
    MTiles<D> t;
    MMerge<D> m;
  } u;
  int32_t pages[kMaxPagesPerSplit];
  int err;
  int badw[kMWaves];  // per wave: a page id of the split out of range
};

__device__ __forceinline__ bf16x8_t as_bf16x8(u32x4_t v) { return __builtin_bit_cast(bf16x8_t, v); }

// chunk-column swizzle of K row r: x ^ (x >> 2) is one-to-one on 4 bits, so
// the 16 rows one MFMA operand read touches land in 16 different 16-byte
// bank groups, and so do the rows 4 apart that one staging store touches
__device__ __forceinline__ int kswz(int r, int mask) { return (r ^ (r >> 2)) & mask; }

// R128: 128 query rows per launch, wave w owning rows 16w .. 16w+15 and
// working through both 32-token halves of every staged tile itself (no team
// merge); otherwise 64 rows, the two teams splitting the tile's tokens.
// One workgroup's split: launched as attn_mfma_kernel with (sp, h, s) =
// the block indices, or as the prefix side of the one-launch cascade.
template <int D>
struct MfmaStore {
  MLds<D> m;
};

template <int D, bool R128, bool PAGE32, class Store = MfmaStore<D>>
__device__ __forceinline__ void mfma_partial(const ValuArgs& a, const int sp, const int h, const int s) {
  MLds<D>& sh = g_lds<Store>.m;
  using C = MCfg<D>;
  constexpr int TPT = C::TPT;
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int r16 = lane & 15, g = lane >> 4;
  const int team = R128 ? 0 : wave >> 2, rb = R128 ? wave : wave & 3;
  const int P = a.page_size;

  // split sp owns pages [sp*base + min(sp, rem), ...) of the plan, base and
  // rem computed on the host (balanced to within one page)
  const int pg0 = a.pg_begin + sp * a.split_base + min(sp, a.split_rem);
  const int npg_plan = a.split_base + (sp < a.split_rem ? 1 : 0);
  const int pg1_plan = pg0 + npg_plan;
  const int32_t* pt_row = a.page_table + static_cast<size_t>(s) * a.max_pages;
  // Setup loads, none under a branch: first the scalar ones (the length and,
  // when pages hold a multiple of 32 tokens so that the 32 tokens a wave
  // stages lie in one page, the page ids of this wave's part of the first two
  // stages), then the small vector loads (this thread's page id of the split,
  // the q rows); the scalar values are waited for after both have gone out,
  // and the first stages' K/V loads follow, so no wait on a small load ever
  // has to wait for K/V too.
  int pidA = 0, pidB = 0;
  __builtin_amdgcn_sched_barrier(0);
  if constexpr (PAGE32) {
    const int half = wave >> 2;
    pidA = pt_row[min(pg0 + (half * kMTeamTok) / P, a.max_pages - 1)];
    pidB = pt_row[min(pg0 + (kMTile + half * kMTeamTok) / P, a.max_pages - 1)];
  }
  const int L_mem = a.seq_lens[s];  // (the prefix pass passes the batch's lengths too, unused)
  __builtin_amdgcn_sched_barrier(0);
  // page ids of the split, one per thread (npg_plan <= kMaxPagesPerSplit =
  // blockDim.x; the index clamped so that the load needs no branch), written
  // to LDS after the first stages' loads have gone out
  const int pt_raw = pt_row[min(pg0 + min(tid, max(npg_plan - 1, 0)), a.max_pages - 1)];

  // q rows of this wave as the B operand of S^T = K Q^T: lane (r16, g) holds
  // row 16*rb + r16, dims 32*ks + 8g .. +8 (zero for padding rows)
  const int row = a.row_base + 16 * rb + r16;
  const bool row_ok = row < a.rows;
  // prefix pass: the launch's rows are those of every sequence of the batch
  const int s_row = a.batch_rows > 0 ? (row_ok ? row : 0) / a.batch_rows : s;
  const int rr = a.batch_rows > 0 ? (row_ok ? row : 0) % a.batch_rows : row;  // row within its sequence
  const bool wave_active = a.row_base + 16 * rb < a.rows;  // uniform: any row of this wave real
  u32x4_t qraw[C::KS];
  {
    const int rc = row_ok ? rr : 0;
    const uint16_t* qp = a.q + ((static_cast<size_t>(s_row) * a.q_len + rc / a.G) * a.H_q + h * a.G + rc % a.G) * D;
#pragma unroll
    for (int ks = 0; ks < C::KS; ++ks) qraw[ks] = *reinterpret_cast<const u32x4_t*>(qp + 32 * ks + 8 * g);
  }
  __builtin_amdgcn_sched_barrier(0);
  // the scalar results are needed from here on (an empty asm that reads them
  // keeps their loads up at the top instead of next to their first use)
  asm volatile("" ::"s"(pidA), "s"(pidB), "s"(L_mem));
  const int L = a.fixed_len >= 0 ? a.fixed_len : L_mem;
  // (a suffix pass also needs every query to see the whole prefix before
  // pg_begin; a length past the plan's pages would leave tokens no split reads)
  const bool bad_len = a.fixed_len < 0 && (L - a.q_len < a.pg_begin * P || L < a.q_len || L > a.max_pages * P ||
                                           L > (a.pg_begin + a.n_pages_plan) * P);
  const int n_pages = bad_len ? 0 : (L + P - 1) / P;
  const int npg = max(min(pg1_plan, n_pages) - pg0, 0);
  const int tok0 = pg0 * P;
  const int tok_end = npg > 0 ? min((pg0 + npg) * P, L) : tok0;  // this split's tokens: [tok0, tok_end)
  const int n_it = (tok_end - tok0 + kMTile - 1) / kMTile;
  int errs = (bad_len && tid == 0) ? HAD_DERR_SEQLEN : 0;

  // visible keys of this lane's row (causal inside the draft; a prefix pass
  // sees the whole prefix)
  const int lim = (row_ok && a.fixed_len < 0) ? (L - a.q_len + rr / a.G + 1) : L;
  const int vis_all = min(tok_end, a.fixed_len >= 0 ? L : L - a.q_len + 1);  // below this: every row, every split token

  // staging map: wave w moves tokens of team w/4, chunk columns
  // CPW*(w%4) .. +CPW; lane -> (token group lu, chunk column lc)
  const int lu = lane % C::GPT;
  const int lc = (wave & 3) * C::CPW + lane / C::GPT;
  const int ltok = (wave >> 2) * kMTeamTok + lu * TPT;  // first tile row of the group
  const int last_tok = max(tok_end - 1, tok0);
  const int last_pg = max(npg - 1, 0);

  // every staging load is unconditional: tokens past the split clamp to its
  // last token, so the addresses stay in bounds and the compiler can count
  // the loads in flight exactly.  A wave stages 32 consecutive tokens; when
  // pages hold a multiple of 32 tokens they lie in one page, and the loads
  // are buffer loads over that (page, KV head) block: a stage past the
  // split's last one (the loop's trailing prefetches) covers 0 bytes and
  // returns zeros without a memory request.  Otherwise every lane addresses
  // its own page.
  auto load_pid = [&](u32x4_t (&kr)[TPT], u32x4_t (&vr)[TPT], int it, int pid) __attribute__((always_inline)) {
    const int t0 = min(tok0 + it * kMTile + ltok, last_tok);
    if constexpr (PAGE32) {
      const int pu = __builtin_amdgcn_readfirstlane(pid < 0 ? 0 : pid);
      const int nbytes = __builtin_amdgcn_readfirstlane(it < n_it ? P * D * 2 : 0);
      const size_t blk = (static_cast<size_t>(pu) * a.H_kv + h) * P * D;
      const __amdgpu_buffer_rsrc_t kr_ = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(a.k_pool + blk), 0,
                                                                           nbytes, kBufferRsrcWord3);
      const __amdgpu_buffer_rsrc_t vr_ = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(a.v_pool + blk), 0,
                                                                           nbytes, kBufferRsrcWord3);
#pragma unroll
      for (int i = 0; i < TPT; ++i) {
        const int t = min(t0 + i, last_tok) % P;
        // non-temporal: the context streams through once per launch (as in the VALU kernel)
        const int off = (t * D + lc * 8) * 2;
        kr[i] = __builtin_amdgcn_raw_buffer_load_b128(kr_, off, 0, kBufferNT);
        vr[i] = __builtin_amdgcn_raw_buffer_load_b128(vr_, off, 0, kBufferNT);
      }
    } else {
      const int pl = pid < 0 ? 0 : pid;
      const uint16_t* kb = a.k_pool + (static_cast<size_t>(pl) * a.H_kv + h) * P * D + lc * 8;
      const uint16_t* vb = a.v_pool + (static_cast<size_t>(pl) * a.H_kv + h) * P * D + lc * 8;
#pragma unroll
      for (int i = 0; i < TPT; ++i) {
        const int t = min(t0 + i, last_tok) % P;  // the group never leaves its page (P % TPT == 0)
        kr[i] = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(kb + t * D));
        vr[i] = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(vb + t * D));
      }
    }
    __builtin_amdgcn_sched_barrier(0);
  };
  auto load = [&](u32x4_t (&kr)[TPT], u32x4_t (&vr)[TPT], int it) __attribute__((always_inline)) {
    const int t0 = min(tok0 + it * kMTile + ltok, last_tok);
    load_pid(kr, vr, it, sh.pages[min(t0 / P - pg0, last_pg)]);
  };

  // The first stages' loads go out before the setup barrier, their page ids
  // read from the page table itself (an id out of range reads page 0; the
  // staging below zeroes what the checked list marks invalid): with PAGE32
  // both stages from the scalar ids read at the start, otherwise the first
  // from a per-lane id and the second after the barrier.
  u32x4_t kA[TPT], vA[TPT], kB[TPT], vB[TPT];
  if constexpr (PAGE32) {
    load_pid(kA, vA, 0, (pidA >= 0 && pidA < a.num_pages) ? pidA : 0);
    load_pid(kB, vB, 1, (pidB >= 0 && pidB < a.num_pages) ? pidB : 0);
  } else {
    const int t0 = min(tok0 + ltok, last_tok);
    const int pid = pt_row[min(pg0 + min(t0 / P - pg0, last_pg), a.max_pages - 1)];
    load_pid(kA, vA, 0, (pid >= 0 && pid < a.num_pages) ? pid : 0);
  }
  // (entry 0 always written, so the clamped loads of an empty split still
  // read a valid page; bad ids become -1 and read page 0)
  if (tid == 0) sh.err = 0;
  if (tid < max(npg_plan, 1)) {
    const int pt_val = tid < npg_plan ? pt_raw : -1;
    const bool ok = pt_val >= 0 && pt_val < a.num_pages;
    if (!ok && tid < npg) errs |= HAD_DERR_PAGE;
    sh.pages[tid] = ok ? pt_val : -1;
  }
  {
    const bool wb = __any(errs & HAD_DERR_PAGE);
    if (lane == 0) sh.badw[wave] = wb;
  }
  u32x4_t qb[C::KS];
#pragma unroll
  for (int ks = 0; ks < C::KS; ++ks) qb[ks] = row_ok ? qraw[ks] : u32x4_t{0u, 0u, 0u, 0u};
  __syncthreads();
  // the scores of tokens on a page whose id is out of range are dropped (its
  // K was read from page 0, its V staged as zeros)
  int any_bad = 0;
#pragma unroll
  for (int w = 0; w < kMWaves; ++w) any_bad |= sh.badw[w];

  auto stage = [&](const u32x4_t (&kr)[TPT], const u32x4_t (&vr)[TPT], int it, int b) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < TPT; ++i) {
      const int r = ltok + i;
      sh.u.t.k[b][r * C::CPR + (lc ^ kswz(r, C::SWZ))] = kr[i];
    }
    // V rows that must not count (past the split, unchecked page) are
    // staged as zeros so stale bits never meet a zero probability
    const int tg = tok0 + it * kMTile + ltok;
    const bool pg_ok = tg < tok_end && sh.pages[min(tg / P - pg0, last_pg)] >= 0;
    u32x4_t v[TPT];
#pragma unroll
    for (int i = 0; i < TPT; ++i) v[i] = (pg_ok && tg + i < tok_end) ? vr[i] : u32x4_t{0u, 0u, 0u, 0u};
    uint16_t* vt = &sh.u.t.vt[b][ltok / kMTeamTok][(8 * lc) * C::VTP + lu * TPT];
#pragma unroll
    for (int j = 0; j < 4; ++j) {  // word j holds d = 8 lc + 2j (low half) and 8 lc + 2j + 1 (high half)
      uint16_t* lo_row = vt + (2 * j) * C::VTP;
      uint16_t* hi_row = vt + (2 * j + 1) * C::VTP;
      if constexpr (TPT == 4) {
        const uint32_t l01 = perm_b32(v[1][j], v[0][j], 0x05040100u);
        const uint32_t l23 = perm_b32(v[3][j], v[2][j], 0x05040100u);
        const uint32_t h01 = perm_b32(v[1][j], v[0][j], 0x07060302u);
        const uint32_t h23 = perm_b32(v[3][j], v[2][j], 0x07060302u);
        *reinterpret_cast<uint2*>(lo_row) = make_uint2(l01, l23);
        *reinterpret_cast<uint2*>(hi_row) = make_uint2(h01, h23);
      } else if constexpr (TPT == 2) {
        *reinterpret_cast<uint32_t*>(lo_row) = perm_b32(v[1][j], v[0][j], 0x05040100u);
        *reinterpret_cast<uint32_t*>(hi_row) = perm_b32(v[1][j], v[0][j], 0x07060302u);
      } else {
        *lo_row = static_cast<uint16_t>(v[0][j] & 0xffffu);
        *hi_row = static_cast<uint16_t>(v[0][j] >> 16);
      }
    }
  };

  f32x4_t o[C::MB];
#pragma unroll
  for (int mb = 0; mb < C::MB; ++mb) o[mb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY, l_run = 0.f;

  auto compute_half = [&](int it, int b, int tm) __attribute__((always_inline)) {
    const u32x4_t* kt = sh.u.t.k[b];
    const uint16_t* vt = sh.u.t.vt[b][tm];
    // ---- S^T for the team's 32 tokens: two 16-token blocks, KS k-steps each
    float sc[8];
#pragma unroll
    for (int tb = 0; tb < 2; ++tb) {
      f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
      const int r = tm * kMTeamTok + 16 * tb + r16;  // A-operand row = token
      const int sw = kswz(r, C::SWZ);
#pragma unroll
      for (int ks = 0; ks < C::KS; ++ks) {
        const u32x4_t kv = kt[r * C::CPR + ((4 * ks + g) ^ sw)];
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(kv), as_bf16x8(qb[ks]), acc, 0, 0, 0);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) sc[4 * tb + i] = acc[i] * a.scale_log2;
    }
    // tokens of slot i: tau(g, i) = 4g + i and 16 + 4g + i - 4 (the mask is
    // skipped for tiles every row sees in full)
    const int pos0 = tok0 + it * kMTile + tm * kMTeamTok;
    if (pos0 + kMTeamTok > vis_all || any_bad) {
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int pos = pos0 + (i < 4 ? 4 * g + i : 16 + 4 * g + (i - 4));
        bool drop = pos >= tok_end || pos >= lim;
        if (any_bad && !drop) drop = sh.pages[min((pos - tok0) / P, last_pg)] < 0;
        if (drop) sc[i] = -INFINITY;
      }
    }

    // ---- online softmax for this lane's row (4 lanes per row: g = 0..3).
    // The reference m_run moves only when a score exceeds it by more than
    // 2^8 (base 2), so p = 2^(s - m_run) <= 256 and the O^T rescale is rare;
    // o, l and m stay consistent, which is all the merge needs.
    float mt = sc[0];
#pragma unroll
    for (int i = 1; i < 8; ++i) mt = fmaxf(mt, sc[i]);
    mt = fmaxf(mt, shfl_xor_f(mt, 16));
    mt = fmaxf(mt, shfl_xor_f(mt, 32));
    const bool move = mt > m_run + 8.f;
    const float m_new = move ? mt : m_run;
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
    if (__any(move)) {
#pragma unroll
      for (int mb = 0; mb < C::MB; ++mb) o[mb] = o[mb] * alpha;
    }
    m_run = m_new;
    const u32x4_t pb = {pw[0], pw[1], pw[2], pw[3]};

    // ---- O^T += V^T P^T over the 32 tokens, one MFMA per 16 output dims
#pragma unroll
    for (int mb = 0; mb < C::MB; ++mb) {
      const uint16_t* vrow = vt + (16 * mb + r16) * C::VTP;
      const uint2 lo = *reinterpret_cast<const uint2*>(vrow + 4 * g);
      const uint2 hi = *reinterpret_cast<const uint2*>(vrow + 16 + 4 * g);
      const u32x4_t va = {lo.x, lo.y, hi.x, hi.y};
      o[mb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(va), as_bf16x8(pb), o[mb], 0, 0, 0);
    }
  };
  auto compute = [&](int it, int b) __attribute__((always_inline)) {
    if (!wave_active) return;
    if constexpr (R128) {
      compute_half(it, b, 0);
      compute_half(it, b, 1);
    } else {
      compute_half(it, b, team);
    }
  };

  // ---- main loop: register stages A (even tiles) and B (odd tiles), LDS
  // buffer 0 for A and 1 for B; the loop exits only at its header
  if constexpr (!PAGE32) load(kB, vB, 1);
  int it = 0;
  while (it + 1 < n_it) {
    stage(kA, vA, it, 0);
    load(kA, vA, it + 2);
    __syncthreads();
    compute(it, 0);
    stage(kB, vB, it + 1, 1);
    load(kB, vB, it + 3);
    __syncthreads();
    compute(it + 1, 1);
    it += 2;
  }
  if (it < n_it) {
    stage(kA, vA, it, 0);
    __syncthreads();
    compute(it, 0);
  }

  // ---- row totals, then team 1 hands its state to team 0 through LDS
  l_run += shfl_xor_f(l_run, 16);
  l_run += shfl_xor_f(l_run, 32);
  if (errs) atomicOr(&sh.err, errs);
  if constexpr (R128) {  // every wave owns its rows outright
    __syncthreads();
    if (tid == 0 && sh.err) set_err(a.d_err, sh.err);
    if (row_ok) {
      const size_t unit = (static_cast<size_t>(s_row) * a.H_kv + h) * a.ns_total + a.split_offset + sp;
      float* op = a.ws_o + (unit * a.ws_rows + rr) * D;
#pragma unroll
      for (int mb = 0; mb < C::MB; ++mb)
        *reinterpret_cast<float4*>(op + 16 * mb + 4 * g) = make_float4(o[mb][0], o[mb][1], o[mb][2], o[mb][3]);
      if (g == 0) {
        a.ws_ml[(unit * a.ws_rows + rr) * 2 + 0] = m_run;
        a.ws_ml[(unit * a.ws_rows + rr) * 2 + 1] = l_run;
      }
    }
    return;
  }
  __syncthreads();  // the tile buffers are free from here on
  if (team == 1 && wave_active) {
    float* orow = sh.u.m.o[rb][r16];
#pragma unroll
    for (int mb = 0; mb < C::MB; ++mb)
      *reinterpret_cast<float4*>(orow + 16 * mb + 4 * g) = make_float4(o[mb][0], o[mb][1], o[mb][2], o[mb][3]);
    if (g == 0) {
      sh.u.m.ml[rb][r16][0] = m_run;
      sh.u.m.ml[rb][r16][1] = l_run;
    }
  }
  __syncthreads();
  if (tid == 0 && sh.err) set_err(a.d_err, sh.err);
  if (team == 0 && row_ok) {
    const float m1 = sh.u.m.ml[rb][r16][0], l1 = sh.u.m.ml[rb][r16][1];
    const float M = fmaxf(m_run, m1);
    const float Ms = (M == -INFINITY) ? 0.f : M;
    const float w0 = exp2f(m_run - Ms), w1 = exp2f(m1 - Ms);
    const float* orow = sh.u.m.o[rb][r16];
    const size_t unit = (static_cast<size_t>(s_row) * a.H_kv + h) * a.ns_total + a.split_offset + sp;
    float* op = a.ws_o + (unit * a.ws_rows + rr) * D;
#pragma unroll
    for (int mb = 0; mb < C::MB; ++mb) {
      const float4 o1 = *reinterpret_cast<const float4*>(orow + 16 * mb + 4 * g);
      *reinterpret_cast<float4*>(op + 16 * mb + 4 * g) =
          make_float4(o[mb][0] * w0 + o1.x * w1, o[mb][1] * w0 + o1.y * w1, o[mb][2] * w0 + o1.z * w1,
                      o[mb][3] * w0 + o1.w * w1);
    }
    if (g == 0) {
      a.ws_ml[(unit * a.ws_rows + rr) * 2 + 0] = M;
      a.ws_ml[(unit * a.ws_rows + rr) * 2 + 1] = l_run * w0 + l1 * w1;
    }
  }
}

}  // namespace

// pages of a multiple of 32 tokens, K and V staged straight into LDS
// (attn_mfma128.hip; called by launch_attn_mfma with the row base and the
// split fields set): dh = 1, rows row_base .. +127; dh = 2 (head_dim >= 128),
// rows row_base .. +63
hipError_t launch_attn_mfma128(const ValuArgs& a, int head_dim, int dh, dim3 grid, hipStream_t stream);

}  // namespace had
