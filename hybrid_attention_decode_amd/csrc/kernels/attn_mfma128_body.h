// Body of the MFMA split-K decode partial for 65..128 query rows per launch
// with pages of a multiple of 32 tokens (e.g. the 128 rows of every sequence
// of a batch that share one prefix, in the prefix pass of cascade decoding:
// 24-ai.news TokenSpeed article, optimisation list, hybrid prefix caching),
// shared by its own kernel (attn_mfma128.hip) and the prefix side of the
// one-launch cascade (attn_cascade.hip).
//
// Same operation and partial format as attn_mfma.hip; the staging and the
// split ranges differ:
//  * Eight waves, two per SIMD, each working through every token of every
//    stage (no team merge).  DH = 1 (up to 128 rows per launch): wave w owns
//    query rows 16w .. 16w+15 and every output dim.  DH = 2 (up to 64 rows):
//    waves w and w + 4 own rows 16w .. 16w+15, each half of the output dims;
//    both form the same scores and softmax state (the same instructions on
//    the same data), so the PV work and its V^T reads are split between them.
//  * K and V go from HBM straight into LDS (buffer loads with the LDS flag:
//    lane l's 16 bytes land at the instruction's LDS base + 16 l), in stages
//    of 32 tokens and kM128Bufs LDS buffers, kM128Bufs - 1 stages in flight;
//    no staging registers and no transposing work in the waves.  A stage
//    lies in one page; its loads are buffer loads over that (page, KV head)
//    block whose size counts only the page's tokens before the split's end,
//    so tokens past the end, a stage past the split's last one and a page
//    whose id is out of range all read as zeros without a memory request.
//  * K row-major with its 16-byte chunks XOR-swizzled by token row (as in
//    attn_mfma.hip); V row-major with two 16-byte pad slots per row: the rows
//    of consecutive tokens start 8 banks apart, so the 8 tokens one
//    transposing read touches per 32 lanes meet on no bank, and the read
//    addresses are a lane base plus constants.
//  * V^T as the A operand of O^T += V^T P^T comes from the transposing LDS
//    read ds_read_b64_tr_b16: within each 16-lane group, lane i receives
//    element i mod 4 of the 8-byte rows addressed by lanes i/4 + 4k (k =
//    0..3).  Lane j = r16 of group g addresses token 4g + j/4 (+16), dims
//    16 mb + 4 (j mod 4) .. +3, so lane i receives dim 16 mb + i of tokens
//    4g + k (+16): the A operand for K indices in the order tau(g, i) of
//    attn_mfma.hip, matching P^T in the layout S^T's accumulators leave.
//  * The stage barrier waits only for this wave's loads of the stage about
//    to be computed (vmcnt) and for LDS operations (lgkmcnt), so the later
//    stages stay in flight across it.
//  * Softmax in base 2 with the scale folded into the exponent's FMA and
//    v_exp_f32 directly (a probability below 2^-126 of the running maximum
//    flushes to zero); row sums of the bf16 probabilities by v_dot2.
#pragma once
#include "attn_mfma_body.h"
#include "prologue_math.h"

namespace had {
namespace {

constexpr int kM128Waves = 8;  // wave w owns query rows 16w .. 16w+15 of the launch
constexpr int kM128Tok = 32;   // tokens per stage
constexpr int kM128Bufs = 4;   // LDS stage buffers

template <int D, int DH>
struct M128Cfg {
  static constexpr int KS = D / 32;                    // QK k-steps (32 d each)
  static constexpr int MB = D / 16 / DH;               // PV output blocks (16 d each) of one wave
  static constexpr int CPR = D / 8;                    // 16-byte chunks per K/V row
  static constexpr int SWZ = (CPR < 16 ? CPR : 16) - 1;
  static constexpr int VP = CPR + 2;                   // V row pitch in 16-byte slots (two pad slots)
  static constexpr int NK = kM128Tok * CPR / 64;       // LDS-load instructions per stage: K
  static constexpr int NV = (kM128Tok * VP + 63) / 64; // ... V (the pad slots included)
  static constexpr int KJ = (NK + kM128Waves - 1) / kM128Waves;  // per wave, at most
  static constexpr int VJ = (NV + kM128Waves - 1) / kM128Waves;
  static_assert((KJ + VJ) * (kM128Bufs - 2) < 64, "vmcnt holds 6 bits");
  static_assert(MB % 4 == 0, "output blocks in groups of four (DH = 2 needs head_dim >= 128)");
};

template <int D>
struct M128Lds {
  u32x4_t k[kM128Bufs][kM128Tok * M128Cfg<D, 1>::CPR];  // [buffer][token][chunk ^ kswz]
  u32x4_t v[kM128Bufs][64 * M128Cfg<D, 1>::NV];         // [buffer][token * VP + chunk]
  int32_t pages[kMaxPagesPerSplit];
  int err;
  int badw[kM128Waves];  // per wave: a page id of the split out of range
  u32x4_t dump[64];      // target of the filler loads that even out the waves' load counts
};

template <int D>
struct M128Store {
  M128Lds<D> m;
};

// The prologue run inline (the layer entry point: QK-RMSNorm, partial
// rotation and gate split of the new tokens; zubnet.ai TokenSpeed article,
// second paragraph).  Every workgroup normalises and rotates its own query
// rows straight into their B-operand registers; the workgroup whose stages
// hold the last position also normalises and rotates the new keys, writes
// the new K/V rows to the pools and adds the new tokens to its partial from
// the copies below (every split's loads stop before the new positions, so
// no workgroup reads a row while it is written).  Extra LDS: cos / sin of
// every new position and rotation pair, the two norm weights, the new rows.
constexpr int kM128New = 8;  // new tokens per sequence, at most

template <int D>
struct M128Pro {
  float cs[kM128New][D / 2];
  float sn[kM128New][D / 2];
  float wq[D];
  float wk[D];
  uint16_t knew[kM128New][D] __attribute__((aligned(16)));
  uint16_t vnew[kM128New][D] __attribute__((aligned(16)));
};

template <int D>
struct M128FusedStore {
  M128Lds<D> m;
  M128Pro<D> f;
};

// One query row in the B-operand layout of S^T = K Q^T (this lane: dims
// 32 ks + 8 g + e, packed bf16 pairs in qb[ks]) normalised with inv and the
// weights w, then rotated below dim 64 HK: pair i = d mod 32 HK, partner in
// k-step ks +- HK of the same lane, cos / sin cs[i], sn[i].  Element by
// element the arithmetic of row_norm_rope_cs (prologue_math.h); only the
// norm's sum of squares runs in this layout's order.
template <int D, int HK>
__device__ __forceinline__ void m128_q_rope(u32x4_t (&qb)[D / 32], float inv, const float* w, const float* cs,
                                            const float* sn, int g) {
  constexpr int KS = D / 32;
  if constexpr (2 * HK <= KS) {
    float y[KS][8];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const uint32_t wd = qb[ks][e / 2];
        const float x = (e & 1) ? bf16_hi(wd) : bf16_lo(wd);
        y[ks][e] = x * inv * w[32 * ks + 8 * g + e];
      }
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      float r[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        r[e] = y[ks][e];
        if constexpr (HK > 0) {
          if (ks < 2 * HK) {
            const int i = 32 * (ks % HK) + 8 * g + e;
            if (ks < HK)
              r[e] = y[ks][e] * cs[i] - y[ks + HK < KS ? ks + HK : KS - 1][e] * sn[i];
            else
              r[e] = y[ks][e] * cs[i] + y[ks >= HK ? ks - HK : 0][e] * sn[i];
          }
        }
      }
      qb[ks] = u32x4_t{pack_bf16x2(r[0], r[1]), pack_bf16x2(r[2], r[3]), pack_bf16x2(r[4], r[5]),
                       pack_bf16x2(r[6], r[7])};
    }
  }
}

typedef __attribute__((address_space(3))) void lds_void_t;
typedef __attribute__((address_space(3))) const char lds_cchar_t;

// s_waitcnt immediate (gfx9 encoding: vmcnt bits 3:0 and 15:14, expcnt 6:4,
// lgkmcnt 11:8; a field at its maximum does not wait)
constexpr int waitcnt_imm(int vm, int lgkm) { return (vm & 15) | ((vm >> 4) << 14) | (7 << 4) | (lgkm << 8); }

// Workgroup barrier over LDS accesses that leaves this wave's LDS loads in
// flight except for the oldest ones (at most VM younger ones outstanding).
// The empty asm statements keep the compiler from moving memory accesses
// across it.
template <int VM>
__device__ __forceinline__ void m128_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(waitcnt_imm(VM, 0));
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// max of three floats.  (Not as inline assembly: the compiler inserts the
// wait states a read of an MFMA result or of a lane swap's outputs needs
// only before instructions it emits itself; a v_max3_f32 written in inline
// assembly right after v_permlane16_swap read stale values in some waves.)
__device__ __forceinline__ float vmax3(float a, float b, float c) { return fmaxf(fmaxf(a, b), c); }

// max over lanes l, l ^ 16, l ^ 32, l ^ 48: v_permlane16_swap exchanges the
// upper 16 lanes of each 32-lane half of its first operand with the lower 16
// of its second, v_permlane32_swap the upper 32 lanes of the first with the
// lower 32 of the second; with both operands x, the two results hold x of
// lane l and of its partner in either order
__device__ __forceinline__ float max_lanes_xor16_32(float x) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = vmax3(__uint_as_float(a[0]), __uint_as_float(a[1]), __uint_as_float(a[1]));
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return vmax3(__uint_as_float(b[0]), __uint_as_float(b[1]), __uint_as_float(b[1]));
}

// V^T operands of eight consecutive output blocks: sixteen transposing
// reads at lo + 32 m and hi + 32 m (m = 0..7), completed before the block
// ends (one LDS round trip for both groups of four)
__device__ __forceinline__ void lds_read_tr8(u32x4_t (&va)[8], const char* lo, const char* hi) {
  const uint32_t alo = static_cast<uint32_t>(reinterpret_cast<uintptr_t>((lds_cchar_t*)lo));
  const uint32_t ahi = static_cast<uint32_t>(reinterpret_cast<uintptr_t>((lds_cchar_t*)hi));
  uint2 l[8], h[8];
  asm volatile(
      "ds_read_b64_tr_b16 %0, %16\n\t"
      "ds_read_b64_tr_b16 %1, %17\n\t"
      "ds_read_b64_tr_b16 %2, %16 offset:32\n\t"
      "ds_read_b64_tr_b16 %3, %17 offset:32\n\t"
      "ds_read_b64_tr_b16 %4, %16 offset:64\n\t"
      "ds_read_b64_tr_b16 %5, %17 offset:64\n\t"
      "ds_read_b64_tr_b16 %6, %16 offset:96\n\t"
      "ds_read_b64_tr_b16 %7, %17 offset:96\n\t"
      "ds_read_b64_tr_b16 %8, %16 offset:128\n\t"
      "ds_read_b64_tr_b16 %9, %17 offset:128\n\t"
      "ds_read_b64_tr_b16 %10, %16 offset:160\n\t"
      "ds_read_b64_tr_b16 %11, %17 offset:160\n\t"
      "ds_read_b64_tr_b16 %12, %16 offset:192\n\t"
      "ds_read_b64_tr_b16 %13, %17 offset:192\n\t"
      "ds_read_b64_tr_b16 %14, %16 offset:224\n\t"
      "ds_read_b64_tr_b16 %15, %17 offset:224\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(l[0]), "=&v"(h[0]), "=&v"(l[1]), "=&v"(h[1]), "=&v"(l[2]), "=&v"(h[2]), "=&v"(l[3]), "=&v"(h[3]),
        "=&v"(l[4]), "=&v"(h[4]), "=&v"(l[5]), "=&v"(h[5]), "=&v"(l[6]), "=&v"(h[6]), "=&v"(l[7]), "=&v"(h[7])
      : "v"(alo), "v"(ahi));
#pragma unroll
  for (int m = 0; m < 8; ++m) va[m] = u32x4_t{l[m].x, l[m].y, h[m].x, h[m].y};
}

// V^T operands of four consecutive output blocks: eight transposing reads,
// at lo + 32 m and hi + 32 m (m = 0..3), completed before the block ends.
// (In inline assembly, so that the compiler adds no wait for the LDS loads
// still in flight into the other stage buffers: with the intrinsic form it
// drains them all first.)
__device__ __forceinline__ void lds_read_tr4(u32x4_t (&va)[4], const char* lo, const char* hi) {
  const uint32_t alo = static_cast<uint32_t>(reinterpret_cast<uintptr_t>((lds_cchar_t*)lo));
  const uint32_t ahi = static_cast<uint32_t>(reinterpret_cast<uintptr_t>((lds_cchar_t*)hi));
  uint2 l0, l1, l2, l3, h0, h1, h2, h3;
  asm volatile(
      "ds_read_b64_tr_b16 %0, %8\n\t"
      "ds_read_b64_tr_b16 %1, %9\n\t"
      "ds_read_b64_tr_b16 %2, %8 offset:32\n\t"
      "ds_read_b64_tr_b16 %3, %9 offset:32\n\t"
      "ds_read_b64_tr_b16 %4, %8 offset:64\n\t"
      "ds_read_b64_tr_b16 %5, %9 offset:64\n\t"
      "ds_read_b64_tr_b16 %6, %8 offset:96\n\t"
      "ds_read_b64_tr_b16 %7, %9 offset:96\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(l0), "=&v"(h0), "=&v"(l1), "=&v"(h1), "=&v"(l2), "=&v"(h2), "=&v"(l3), "=&v"(h3)
      : "v"(alo), "v"(ahi));
  va[0] = u32x4_t{l0.x, l0.y, h0.x, h0.y};
  va[1] = u32x4_t{l1.x, l1.y, h1.x, h1.y};
  va[2] = u32x4_t{l2.x, l2.y, h2.x, h2.y};
  va[3] = u32x4_t{l3.x, l3.y, h3.x, h3.y};
}

// One workgroup's split: launched as attn_mfma128_kernel with (sp, h, s) =
// the block indices, or as the prefix side of the one-launch cascade.  For
// this body a.split_base and a.split_rem count 32-token stages of the plan
// (its n_pages_plan pages from pg_begin), not pages: split sp takes stages
// sp * base + min(sp, rem) .. + base (+1 while sp < rem), so the splits are
// balanced to within one stage and a split may start and end inside a page.
// FUSED: the prologue inline (Store = M128FusedStore<D>, inputs in f; a.q
// unused), for the rows of one launch (row_base 0) and q_len <= kM128New,
// with R = 0, 64 or a multiple of 128 (the host checks).
template <int D, int DH, class Store = M128Store<D>, bool FUSED = false>
__device__ __forceinline__ void mfma128_partial(const ValuArgs& a, const int sp, const int h, const int s,
                                                const FusedArgs& f = FusedArgs{}) {
  static_assert(DH == 1 || DH == 2, "rows per wave group");
  M128Lds<D>& sh = g_lds<Store>.m;
  using C = M128Cfg<D, DH>;
  constexpr int NRG = kM128Waves / DH;  // row groups of 16
  constexpr int NB = kM128Bufs;
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int r16 = lane & 15, g = lane >> 4;
  const int rg = wave % NRG, dh = wave / NRG;  // row group, part of the output dims
  const int P = a.page_size;

  // this split's stages of the plan and the pages they touch
  const int st0 = sp * a.split_base + min(sp, a.split_rem);
  const int nst = a.split_base + (sp < a.split_rem ? 1 : 0);
  const int tok0 = a.pg_begin * P + kM128Tok * st0;        // first token of the split
  const int tok_plan_end = tok0 + kM128Tok * nst;          // ... past its last (plan)
  const int pg0 = tok0 / P;                                // its first page
  const int off0 = tok0 - pg0 * P;                         // token offset of the split in that page
  const int npg_plan = nst > 0 ? (tok_plan_end - 1) / P - pg0 + 1 : 0;  // pages the plan's range touches
  const int32_t* pt_row = a.page_table + static_cast<size_t>(s) * a.max_pages;
  // setup: scalar loads first (length, page ids of the first NB - 1
  // stages), then the small vector loads (this thread's page id of the
  // split, the q rows), then the LDS loads of the first stages
  __builtin_amdgcn_sched_barrier(0);
  int pid0[NB - 1];
#pragma unroll
  for (int r = 0; r < NB - 1; ++r) pid0[r] = pt_row[min(pg0 + (off0 + r * kM128Tok) / P, a.max_pages - 1)];
  const int L_mem = a.seq_lens[s];
  __builtin_amdgcn_sched_barrier(0);
  static_assert(64 * kM128Waves >= kMaxPagesPerSplit, "a split's page ids are read one per thread");
  const int pt_raw = pt_row[min(pg0 + min(tid, max(npg_plan - 1, 0)), a.max_pages - 1)];

  // q rows of this wave as the B operand of S^T = K Q^T: lane (r16, g)
  // holds row 16 wave + r16, dims 32 ks + 8 g .. +8 (zero for padding rows)
  const int row = a.row_base + 16 * rg + r16;
  const bool row_ok = row < a.rows;
  // prefix pass: the launch's rows are those of every sequence of the batch
  const int s_row = a.batch_rows > 0 ? (row_ok ? row : 0) / a.batch_rows : s;
  const int rr = a.batch_rows > 0 ? (row_ok ? row : 0) % a.batch_rows : row;  // row within its sequence
  const bool wave_active = a.row_base + 16 * rg < a.rows;                     // uniform
  u32x4_t qb[C::KS];
  {
    const int rc = row_ok ? rr : 0;
    const size_t hd = (static_cast<size_t>(s_row) * a.q_len + rc / a.G) * a.H_q + h * a.G + rc % a.G;
    // (fused: the raw row, the q half of qg)
    const uint16_t* qp = FUSED ? f.qg + hd * 2 * D : a.q + hd * D;
#pragma unroll
    for (int ks = 0; ks < C::KS; ++ks) qb[ks] = *reinterpret_cast<const u32x4_t*>(qp + 32 * ks + 8 * g);
  }
  // fused: the norm weights (a float4 per thread, staged through LDS), the
  // raw K/V row of new token min(wave, q_len - 1) (lane l: dims l + 64 m),
  // and this split's share of the gate block of the launch's rows (16-byte
  // chunks sp, sp + ns, sp + 2 ns, ...: every split copies a few, rather
  // than every split loading the whole block for split 0 to copy) -- all
  // unconditional, indexes clamped
  constexpr int E = D / 64;
  constexpr int NGC = (16 * NRG) * (D / 8) / (64 * kM128Waves);  // gate chunks per thread, at most
  static_assert(NGC >= 1 && (16 * NRG) * (D / 8) % (64 * kM128Waves) == 0, "gate chunks cover the rows");
  [[maybe_unused]] float4 w_st{};
  [[maybe_unused]] uint16_t k_raw[E], v_raw[E];
  [[maybe_unused]] u32x4_t gate_ch[NGC];
  if constexpr (FUSED) {
    w_st = reinterpret_cast<const float4*>(tid < D / 4 ? f.w_q : f.w_k)[tid % (D / 4)];
    const size_t kr = ((static_cast<size_t>(s) * a.q_len + min(wave, a.q_len - 1)) * a.H_kv + h) * D;
#pragma unroll
    for (int m = 0; m < E; ++m) {
      k_raw[m] = f.k_new[kr + lane + 64 * m];
      v_raw[m] = f.v_new[kr + lane + 64 * m];
    }
#pragma unroll
    for (int c = 0; c < NGC; ++c) {
      const int ch = min(sp + a.num_splits * (tid + 64 * kM128Waves * c), a.rows * (D / 8) - 1);
      const int r = ch / (D / 8);
      const size_t hd = (static_cast<size_t>(s) * a.q_len + r / a.G) * a.H_q + h * a.G + r % a.G;
      gate_ch[c] = *reinterpret_cast<const u32x4_t*>(f.qg + hd * 2 * D + D + 8 * (ch % (D / 8)));
    }
  }
  __builtin_amdgcn_sched_barrier(0);
  // the scalar results are needed from here on
#pragma unroll
  for (int r = 0; r < NB - 1; ++r) asm volatile("" ::"s"(pid0[r]));
  asm volatile("" ::"s"(L_mem));
  const int L = a.fixed_len >= 0 ? a.fixed_len : L_mem;
  // (a suffix pass also needs every query to see the whole prefix before
  // pg_begin; a length past the plan's pages would leave tokens no split reads)
  const bool bad_len = a.fixed_len < 0 && (L - a.q_len < a.pg_begin * P || L < a.q_len || L > a.max_pages * P ||
                                           L > (a.pg_begin + a.n_pages_plan) * P);
  // fused: the loads stop before the new positions, and the split whose
  // stages hold the last position owns the new tokens
  const int kv_end = FUSED ? L - a.q_len : L;
  const bool own = FUSED && !bad_len && L - 1 >= tok0 && L - 1 < tok_plan_end;
  const int tok_end = bad_len ? tok0 : max(min(tok_plan_end, kv_end), tok0);  // this split's tokens: [tok0, tok_end)
  const int npg = tok_end > tok0 ? (tok_end - 1) / P - pg0 + 1 : 0;     // pages holding them
  const int n_it = (tok_end - tok0 + kM128Tok - 1) / kM128Tok;
  int errs = (bad_len && tid == 0) ? HAD_DERR_SEQLEN : 0;
  // visible keys of this lane's row (causal inside the draft; a prefix pass
  // sees the whole prefix), and the bound below which every row sees every
  // split token
  const int lim = FUSED ? kv_end : (row_ok && a.fixed_len < 0) ? (L - a.q_len + rr / a.G + 1) : L;
  const int vis_all = min(tok_end, FUSED ? kv_end : a.fixed_len >= 0 ? L : L - a.q_len + 1);
  const int last_pg = max(npg - 1, 0);

  // LDS loads of stage it into buffer b, page id pid (-1: out of range),
  // page pg_rel of the split, t_tok tokens into it.  The stage's NK K and
  // NV V instructions go round the waves; lane l of instruction j fills
  // slot 64 j + l: for K token row (64 j + l) / CPR, slot column x = l mod
  // CPR, holding the chunk the swizzle puts there; for V token row
  // (64 j + l) / VP, chunk (64 j + l) mod VP, the pad slots loaded from past
  // the buffer's end (zeros, no memory request).  Every wave issues KJ + VJ
  // instructions, those past NK or NV fillers of the same kind into the
  // dump slots, so one fixed vmcnt bound serves every wave.  Byte offsets
  // within the stage's first token row are fixed per lane.
  constexpr int kPastEnd = 0x40000000;  // beyond any (page, head) block
  int kofs_dma[C::KJ], vofs_dma[C::VJ];
#pragma unroll
  for (int i = 0; i < C::KJ; ++i) {
    const int sl = 64 * (wave + kM128Waves * i) + lane;
    const int r = sl / C::CPR, xk = sl % C::CPR;
    kofs_dma[i] = wave + kM128Waves * i < C::NK ? r * D * 2 + (xk ^ kswz(r, C::SWZ)) * 16 : kPastEnd;
  }
#pragma unroll
  for (int i = 0; i < C::VJ; ++i) {
    const int sl = 64 * (wave + kM128Waves * i) + lane;
    const int r = sl / C::VP, xv = sl % C::VP;
    vofs_dma[i] = (wave + kM128Waves * i < C::NV && xv < C::CPR) ? r * D * 2 + xv * 16 : kPastEnd;
  }
  auto issue = [&](int it, int b, int pid, int pg_rel, int t_tok) __attribute__((always_inline)) {
    const int pg_tok0 = (pg0 + pg_rel) * P;
    const int valid = (pid >= 0 && it < n_it) ? min(max(tok_end - pg_tok0, 0), P) : 0;  // tokens that count
    const int nbytes = __builtin_amdgcn_readfirstlane(valid * D * 2);
    const int pu = __builtin_amdgcn_readfirstlane(pid < 0 ? 0 : pid);
    const size_t blk = (static_cast<size_t>(pu) * a.H_kv + h) * P * D;
    const __amdgpu_buffer_rsrc_t kr_ = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(a.k_pool + blk), 0,
                                                                         nbytes, kBufferRsrcWord3);
    const __amdgpu_buffer_rsrc_t vr_ = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(a.v_pool + blk), 0,
                                                                         nbytes, kBufferRsrcWord3);
    const int t_bytes = t_tok * D * 2;  // first token of the stage within its page
    // non-temporal: the context streams through once per launch
#pragma unroll
    for (int i = 0; i < C::KJ; ++i) {
      const int j = wave + kM128Waves * i;
      u32x4_t* dst = (C::NK % kM128Waves == 0 || j < C::NK) ? &sh.k[b][64 * j] : sh.dump;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(kr_, (lds_void_t*)dst, 16, t_bytes + kofs_dma[i], 0, 0, kBufferNT);
    }
#pragma unroll
    for (int i = 0; i < C::VJ; ++i) {
      const int j = wave + kM128Waves * i;
      u32x4_t* dst = (C::NV % kM128Waves == 0 || j < C::NV) ? &sh.v[b][64 * j] : sh.dump;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(vr_, (lds_void_t*)dst, 16, t_bytes + vofs_dma[i], 0, 0, kBufferNT);
    }
  };

  // first stages from the scalar page ids; (nx_pg, nx_off) steps through
  // the stages' pages and token offsets (a page holds a whole number of
  // stages, and a split starts on a stage)
  int nx_pg = 0, nx_off = off0;
  auto step = [&]() __attribute__((always_inline)) {
    nx_off += kM128Tok;
    if (nx_off == P) {
      nx_off = 0;
      ++nx_pg;
    }
  };
  // (fused: only the first stage before the setup barrier -- the setup's
  // small loads of the raw q rows, the gate block and the weights return
  // sooner behind a smaller burst -- and the others right after it)
  constexpr int NE = FUSED ? 1 : NB - 1;
#pragma unroll
  for (int r = 0; r < NE; ++r) {
    issue(r, r, (pid0[r] >= 0 && pid0[r] < a.num_pages) ? pid0[r] : -1, nx_pg, nx_off);
    step();
  }
  if (tid == 0) sh.err = 0;
  // the checked page list (bad ids become -1)
  if (tid < max(npg_plan, 1)) {
    const int pv = tid < npg_plan ? pt_raw : -1;
    const bool pok = pv >= 0 && pv < a.num_pages;
    if (!pok && tid < npg) errs |= HAD_DERR_PAGE;
    sh.pages[tid] = pok ? pv : -1;
  }
  {
    const bool wb = __any(errs & HAD_DERR_PAGE);
    if (lane == 0) sh.badw[wave] = wb;
  }
  if constexpr (FUSED) {
    // cos / sin of pair i at new position t, and the norm weights -> LDS
    M128Pro<D>& F = g_lds<Store>.f;
    const int half = f.R / 2;
    for (int e = tid; e < a.q_len * half; e += 64 * kM128Waves) {
      const int t = e / half, i = e - t * half;
      rope_cs(L - a.q_len + t, i, f.rope_coef, F.cs[t][i], F.sn[t][i]);
    }
    if (tid < D / 2) *reinterpret_cast<float4*>((tid < D / 4 ? F.wq : F.wk) + 4 * (tid % (D / 4))) = w_st;
  }
#pragma unroll
  for (int ks = 0; ks < C::KS; ++ks) qb[ks] = row_ok ? qb[ks] : u32x4_t{0u, 0u, 0u, 0u};
  m128_barrier<63>();  // the page list is in LDS; the first stages stay in flight
#pragma unroll
  for (int r = NE; r < NB - 1; ++r) {
    issue(r, r, (pid0[r] >= 0 && pid0[r] < a.num_pages) ? pid0[r] : -1, nx_pg, nx_off);
    step();
  }
  // the scores of a stage whose page id is out of range are dropped (its K
  // and V read as zeros)
  int any_bad = 0;
#pragma unroll
  for (int w = 0; w < kM128Waves; ++w) any_bad |= sh.badw[w];
  if constexpr (FUSED) {
    M128Pro<D>& F = g_lds<Store>.f;
    // this lane's query row: RMSNorm over the four lanes of the row, rotation
    const int jq = (row_ok ? rr : 0) / a.G;
    float ss = 0.f;
#pragma unroll
    for (int ks = 0; ks < C::KS; ++ks)
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        const float lo = bf16_lo(qb[ks][w]), hi = bf16_hi(qb[ks][w]);
        ss += lo * lo;
        ss += hi * hi;
      }
    ss = sum_xor32(sum_xor16(ss));
    const float inv = 1.f / sqrtf(ss / static_cast<float>(D) + f.eps);
    const float* cs = F.cs[min(jq, kM128New - 1)];
    const float* sn = F.sn[min(jq, kM128New - 1)];
    switch (f.R / 64) {  // k-steps between rotation partners (R = 0, 64, 128 or 256)
      case 0: m128_q_rope<D, 0>(qb, inv, F.wq, cs, sn, g); break;
      case 1: m128_q_rope<D, 1>(qb, inv, F.wq, cs, sn, g); break;
      case 2: m128_q_rope<D, 2>(qb, inv, F.wq, cs, sn, g); break;
      default: m128_q_rope<D, 4>(qb, inv, F.wq, cs, sn, g); break;
    }
#pragma unroll
    for (int ks = 0; ks < C::KS; ++ks) qb[ks] = row_ok ? qb[ks] : u32x4_t{0u, 0u, 0u, 0u};
    // split 0: q (one wave of each pair) to the optional output; every
    // split: its gate chunks
    if (sp == 0 && f.q_out && row_ok && dh == 0) {
      const size_t hd = (static_cast<size_t>(s) * a.q_len + jq) * a.H_q + h * a.G + rr % a.G;
#pragma unroll
      for (int ks = 0; ks < C::KS; ++ks) *reinterpret_cast<u32x4_t*>(f.q_out + hd * D + 32 * ks + 8 * g) = qb[ks];
    }
#pragma unroll
    for (int c = 0; c < NGC; ++c) {
      const int ch = sp + a.num_splits * (tid + 64 * kM128Waves * c), r = ch / (D / 8);
      if (r < a.rows) {
        const size_t hd = (static_cast<size_t>(s) * a.q_len + r / a.G) * a.H_q + h * a.G + r % a.G;
        *reinterpret_cast<u32x4_t*>(f.gate_out + hd * D + 8 * (ch % (D / 8))) = gate_ch[c];
      }
    }
    // the owner: new key `wave` normalised and rotated (the prologue's own
    // row arithmetic, so the pool rows equal the prologue kernel's bits),
    // into LDS and, with V, into the pools
    if (own && wave < a.q_len) {
      const int pid_new = pt_row[min(L - a.q_len + wave, a.max_pages * P - 1) / P];  // (L >= q_len when own)
      RowIn<D> kin;
      float cs_e[E], sn_e[E];
#pragma unroll
      for (int m = 0; m < E; ++m) {
        const int d = lane + 64 * m;
        kin.x[m] = k_raw[m];
        kin.w[m] = F.wk[d];
        cs_e[m] = 1.f;
        sn_e[m] = 0.f;
        if (64 * m < f.R && d < f.R) {
          cs_e[m] = F.cs[wave][d % (f.R / 2)];
          sn_e[m] = F.sn[wave][d % (f.R / 2)];
        }
      }
      uint16_t y[E];
      row_norm_rope_cs<D>(kin, cs_e, sn_e, f.R, f.eps, nullptr, lane, y);
      const int pos = L - a.q_len + wave;
      const bool pok = pid_new >= 0 && pid_new < a.num_pages;
      const size_t dst = ((static_cast<size_t>(pok ? pid_new : 0) * a.H_kv + h) * P + pos % P) * D;
#pragma unroll
      for (int m = 0; m < E; ++m) {
        F.knew[wave][lane + 64 * m] = y[m];
        F.vnew[wave][lane + 64 * m] = v_raw[m];
        if (pok) {
          f.k_pool[dst + lane + 64 * m] = y[m];
          f.v_pool[dst + lane + 64 * m] = v_raw[m];
        }
      }
      if (!pok && lane == 0) errs |= HAD_DERR_PAGE;
    }
  }

  f32x4_t o[C::MB];
#pragma unroll
  for (int mb = 0; mb < C::MB; ++mb) o[mb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY, l_run = 0.f;
  const float sl2 = a.scale_log2;

  // transposing-read source of this lane: token 4g + r16/4 (+16), chunk
  // 2 mb + (r16 mod 4)/2, 8-byte half r16 mod 2: a lane base plus constants
  const int vlane = ((4 * g + (r16 >> 2)) * C::VP + 2 * C::MB * dh + ((r16 & 3) >> 1)) * 16 + 8 * (r16 & 1);
  // K operand of k-step ks = 4u + q for token block tb: row 16 tb + r16,
  // chunk (4 ks + g) ^ kswz = 4 (4u + (q ^ kh)) + (g ^ kl), kh and kl the
  // swizzle's high and low bits: byte offset koff[tb][q] + 256 u
  constexpr int KQ = C::KS < 4 ? C::KS : 4;
  int koff[2][KQ];
#pragma unroll
  for (int tb = 0; tb < 2; ++tb) {
    const int sw = kswz(16 * tb + r16, C::SWZ);
#pragma unroll
    for (int qq = 0; qq < KQ; ++qq)
      koff[tb][qq] = ((16 * tb + r16) * C::CPR + 4 * (qq ^ (sw >> 2)) + (g ^ (sw & 3))) * 16;
  }

  // Operand reads run ahead of their MFMAs: the K reads of the next KD
  // k-steps; the V^T reads in groups of VG output blocks (eight where the
  // wave's blocks come in eights), the first before the softmax, each later
  // one while the previous group's MFMAs run.
  constexpr int KD = 2;
  constexpr int VG = C::MB % 8 == 0 ? 8 : 4;
  auto compute = [&](int it, int bf) __attribute__((always_inline)) {
    if (!wave_active) return;
    const char* kb = reinterpret_cast<const char*>(sh.k[bf]);
    const char* vb = reinterpret_cast<const char*>(sh.v[bf]) + vlane;
    auto kread = [&](int ks, int tb) __attribute__((always_inline)) {
      return *reinterpret_cast<const u32x4_t*>(kb + koff[tb][ks % KQ] + 256 * (ks / KQ));
    };
    // V^T operands of output blocks VG grp .. VG grp + VG - 1
    auto vread = [&](u32x4_t (&va)[VG], int grp) __attribute__((always_inline)) {
      if constexpr (VG == 8)
        lds_read_tr8(va, vb + 256 * grp, vb + 256 * grp + 16 * C::VP * 16);
      else
        lds_read_tr4(va, vb + 128 * grp, vb + 128 * grp + 16 * C::VP * 16);
    };
    // ---- S^T for both 16-token blocks: two independent accumulation chains
    u32x4_t kr[KD][2];
#pragma unroll
    for (int d = 0; d < KD; ++d) {
      kr[d][0] = kread(d, 0);
      kr[d][1] = kread(d, 1);
    }
    f32x4_t acc0 = {0.f, 0.f, 0.f, 0.f}, acc1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < C::KS; ++ks) {
      const u32x4_t k0 = kr[ks % KD][0], k1 = kr[ks % KD][1];
      if (ks + KD < C::KS) {
        kr[ks % KD][0] = kread(ks + KD, 0);
        kr[ks % KD][1] = kread(ks + KD, 1);
      }
      acc0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(k0), as_bf16x8(qb[ks]), acc0, 0, 0, 0);
      acc1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(k1), as_bf16x8(qb[ks]), acc1, 0, 0, 0);
    }
    u32x4_t vr[VG];
    vread(vr, 0);
    // raw scores; tokens of slot i: tau(g, i) = 4g + i and 16 + 4g + i - 4
    float raw[8];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      raw[i] = acc0[i];
      raw[4 + i] = acc1[i];
    }
    const int pos0 = tok0 + it * kM128Tok;
    const bool pg_bad = any_bad && sh.pages[min((off0 + pos0 - tok0) / P, last_pg)] < 0;  // a stage lies in one page
    if (pos0 + kM128Tok > vis_all || pg_bad) {
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int pos = pos0 + (i < 4 ? 4 * g + i : 16 + 4 * g + (i - 4));
        if (pg_bad || pos >= tok_end || pos >= lim) raw[i] = -INFINITY;
      }
    }
    // ---- online softmax for this lane's row (4 lanes per row), reference
    // moved only when a score exceeds it by more than 2^8 (as attn_mfma.hip)
    const float mr = max_lanes_xor16_32(
        vmax3(vmax3(raw[0], raw[1], raw[2]), vmax3(raw[3], raw[4], raw[5]), vmax3(raw[6], raw[7], raw[7])));
    const float mt = mr * sl2;
    const bool move = mt > m_run + 8.f;
    const float m_new = move ? mt : m_run;
    const float m_sub = (m_new == -INFINITY) ? 0.f : m_new;
    const float alpha = __builtin_amdgcn_exp2f(m_run - m_sub);
    uint32_t pw[4];
    float lsum = 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      pw[i] = pack_bf16x2(__builtin_amdgcn_exp2f(fmaf(raw[2 * i], sl2, -m_sub)),
                          __builtin_amdgcn_exp2f(fmaf(raw[2 * i + 1], sl2, -m_sub)));
      lsum = dot2_bf16(pw[i], 0x3F803F80u, lsum);  // + both bf16 probabilities
    }
    l_run = l_run * alpha + lsum;
    if (__any(move)) {
#pragma unroll
      for (int mb = 0; mb < C::MB; ++mb) o[mb] = o[mb] * alpha;
    }
    m_run = m_new;
    const u32x4_t pb = {pw[0], pw[1], pw[2], pw[3]};
    // ---- O^T += V^T P^T, VG output blocks per group of V^T reads
#pragma unroll
    for (int grp = 0; grp < C::MB / VG; ++grp) {
      if (grp > 0) vread(vr, grp);
#pragma unroll
      for (int m = 0; m < VG; ++m)
        o[VG * grp + m] =
            __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(vr[m]), as_bf16x8(pb), o[VG * grp + m], 0, 0, 0);
    }
  };

  // main loop: wait for this wave's part of stage it (NB - 2 later stages
  // may stay outstanding), barrier (every wave's part has landed, and every
  // wave is done with stage it - 1, whose buffer is refilled next)
  // (the page id of the next stage to issue is read from LDS one iteration
  // ahead)
  int pid_nx = sh.pages[min(nx_pg, last_pg)];
  for (int it = 0; it < n_it; ++it) {
    m128_barrier<(C::KJ + C::VJ) * (NB - 2)>();
    const int nx = it + NB - 1;
    issue(nx, nx % NB, pid_nx, nx_pg, nx_off);
    step();
    pid_nx = sh.pages[min(nx_pg, last_pg)];
    compute(it, it % NB);
  }
  // no LDS load may still be landing when the workgroup ends
  __builtin_amdgcn_s_waitcnt(waitcnt_imm(0, 15));

  // row totals; every wave owns its rows outright
  l_run += shfl_xor_f(l_run, 16);
  l_run += shfl_xor_f(l_run, 32);
  if (errs) atomicOr(&sh.err, errs);
  __syncthreads();
  if (tid == 0 && sh.err) set_err(a.d_err, sh.err);
  if constexpr (FUSED) {
    // the owner adds the new tokens (causal inside the draft: row rr's
    // token rr / G sees new tokens 0 .. rr / G) from the LDS copies; the
    // four lanes of a row form the same scores, so m and l stay row-uniform
    if (own && wave_active) {
      M128Pro<D>& F = g_lds<Store>.f;
      const int jq = (row_ok ? rr : 0) / a.G;
      float sc[kM128New];
      float mx = m_run;
#pragma unroll
      for (int t = 0; t < kM128New; ++t) {
        float dsum = 0.f;
        if (t < a.q_len) {
#pragma unroll
          for (int ks = 0; ks < C::KS; ++ks) {
            const u32x4_t kv = *reinterpret_cast<const u32x4_t*>(&F.knew[t][32 * ks + 8 * g]);
#pragma unroll
            for (int w = 0; w < 4; ++w) dsum = dot2_bf16(qb[ks][w], kv[w], dsum);
          }
          dsum = sum_xor32(sum_xor16(dsum));
        }
        sc[t] = (t < a.q_len && t <= jq) ? dsum * sl2 : -INFINITY;
        mx = fmaxf(mx, sc[t]);
      }
      const float alpha = (m_run == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(m_run - mx);
      float pt[kM128New], lsum = 0.f;
#pragma unroll
      for (int t = 0; t < kM128New; ++t) {
        pt[t] = (sc[t] == -INFINITY) ? 0.f : bf16_to_f32(f32_to_bf16(__builtin_amdgcn_exp2f(sc[t] - mx)));
        lsum += pt[t];
      }
      l_run = l_run * alpha + lsum;
#pragma unroll
      for (int mb = 0; mb < C::MB; ++mb) o[mb] = o[mb] * alpha;
#pragma unroll
      for (int t = 0; t < kM128New; ++t) {
        if (t < a.q_len) {
#pragma unroll
          for (int mb = 0; mb < C::MB; ++mb) {
            const uint2 vv = *reinterpret_cast<const uint2*>(&F.vnew[t][16 * (C::MB * dh + mb) + 4 * g]);
            o[mb][0] += pt[t] * bf16_lo(vv.x);
            o[mb][1] += pt[t] * bf16_hi(vv.x);
            o[mb][2] += pt[t] * bf16_lo(vv.y);
            o[mb][3] += pt[t] * bf16_hi(vv.y);
          }
        }
      }
      m_run = mx;
    }
  }
  if (row_ok) {
    const size_t unit = (static_cast<size_t>(s_row) * a.H_kv + h) * a.ns_total + a.split_offset + sp;
    float* op = a.ws_o + (unit * a.ws_rows + rr) * D + 16 * C::MB * dh;
#pragma unroll
    for (int mb = 0; mb < C::MB; ++mb)
      *reinterpret_cast<float4*>(op + 16 * mb + 4 * g) = make_float4(o[mb][0], o[mb][1], o[mb][2], o[mb][3]);
    if (g == 0 && dh == 0) {
      a.ws_ml[(unit * a.ws_rows + rr) * 2 + 0] = m_run;
      a.ws_ml[(unit * a.ws_rows + rr) * 2 + 1] = l_run;
    }
  }
}

}  // namespace
}  // namespace had
