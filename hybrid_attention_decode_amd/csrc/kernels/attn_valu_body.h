// Body of the VALU split-K decode partial (query rows per KV head < 16),
// shared by its own kernel (attn_valu.hip) and the one-launch cascade
// (attn_cascade.hip).  The operation and the gfx950 mapping are described in
// attn_valu.hip.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "attn_internal.h"
#include "kcommon.h"
#include "prologue_math.h"

namespace had {
namespace {

constexpr int kWaves = 8;
constexpr int kRows = 8;  // rows handled per launch (padded with zero queries)
constexpr int kTT = 8;    // tokens per tile
static_assert(kMaxPagesPerSplit <= 64 * kWaves, "one page-table entry per thread");

template <int D>
struct Cfg {
  static constexpr int LPT = (D == 64) ? 8 : 16;  // lanes per token in QK
  static constexpr int CH = D / (LPT * 8);         // 16-byte K chunks per lane per token
  static constexpr int TPS = 64 / LPT;             // tokens per QK step
  static constexpr int TS = kTT / TPS;             // QK steps per tile
  static constexpr int DPL = 4;                    // d per lane in PV
  static constexpr int TG = 256 / D;               // token groups in PV
  static constexpr int VPL = kTT / TG;             // V rows per lane per tile
  static constexpr int NPAIR = VPL / 2;            // dot2 token pairs per lane per tile
  static_assert(CH >= 1 && TS >= 1 && NPAIR >= 1, "unsupported head_dim");
};

// Lane -> row permutation used by the reduce-scatter: the partners of the
// three DPP levels (j^7, j^2, j^1 inside groups of 8) hold rows differing in
// bit 2, 1 and 0 respectively.
__device__ __forceinline__ int sigma(int j) { return (j & 3) ^ ((j & 4) ? 7 : 0); }

template <int D>
struct Tile {
  uint4 k[Cfg<D>::TS][Cfg<D>::CH];
  uint2 v[Cfg<D>::VPL];
};

struct Lds {
  uint2 q[kRows][64];                // query block (bf16), rows in launch order
  float o[kWaves + 1][kRows][256];  // per-wave partial outputs for the merge (+ the new tokens' when fused)
  float ml[kWaves + 1][kRows][2];   // per-wave (m, l)
  uint16_t knew[kRows][256];         // fused: the new tokens' K rows (bf16, normalised and rotated)
  uint16_t vnew[kRows][256];         // fused: the new tokens' V rows
  uint32_t p[kWaves][4][kRows];     // bf16 p pairs: [pair][row]
  float alpha[kWaves][kRows];       // per-row rescale factor of the current tile
  int32_t pages[kMaxPagesPerSplit];  // page ids of the workgroup's range (-1 = invalid)
  int next;                          // next tile to claim
  int err;                           // HAD_DERR bits seen by the workgroup
};

// K and V of one 8-token tile: page `pid`, tile `tip` inside the page.
// Buffer loads over one (page, KV head) block: a refill past the split's
// last tile passes live = false, its descriptor covers 0 bytes and the loads
// return zeros without a memory request (the wave would otherwise wait for
// a useless 8 KB re-read before it leaves the loop), and no offset can leave
// the block.  The loads carry the non-temporal hint: every K/V byte is read
// once per launch, and streaming the context through the caches would evict
// what the rest of the decode step reuses (recurrent states, page tables,
// the partials the merge reads); measured on the 48-layer step it is also
// the faster stream (1M context: 6.4 instead of 5.8 TB/s).
template <int D>
__device__ __forceinline__ void load_tile_at(Tile<D>& T, const ValuArgs& a, int pid, int tip, bool live, int h, int tg,
                                             int j, int tgv, int dl) {
  using C = Cfg<D>;
  const int pu = __builtin_amdgcn_readfirstlane(pid);
  const int nbytes = __builtin_amdgcn_readfirstlane(live ? a.page_size * D * 2 : 0);
  const size_t blk = (static_cast<size_t>(pu) * a.H_kv + h) * a.page_size * D;
  const __amdgpu_buffer_rsrc_t kr = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(a.k_pool + blk), 0, nbytes,
                                                                      kBufferRsrcWord3);
  const __amdgpu_buffer_rsrc_t vr = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(a.v_pool + blk), 0, nbytes,
                                                                      kBufferRsrcWord3);
  const int t0 = tip * kTT;
#pragma unroll
  for (int i = 0; i < C::TS; ++i)
#pragma unroll
    for (int c = 0; c < C::CH; ++c) {
      const auto x = __builtin_amdgcn_raw_buffer_load_b128(kr, ((t0 + i * C::TPS + tg) * D + (j + c * C::LPT) * 8) * 2,
                                                           0, kBufferNT);
      T.k[i][c] = make_uint4(x[0], x[1], x[2], x[3]);
    }
#pragma unroll
  for (int i = 0; i < C::VPL; ++i) {
    const auto x = __builtin_amdgcn_raw_buffer_load_b64(vr, ((t0 + tgv + C::TG * i) * D + dl * C::DPL) * 2, 0,
                                                        kBufferNT);
    T.v[i] = make_uint2(x[0], x[1]);
  }
}

// One workgroup's split of the partial: launched as attn_valu_kernel with
// (bx, h, bz) the block indices, or as one side of the one-launch cascade.
struct ValuStore {
  Lds v;
};

template <int D, bool FUSED, class Store = ValuStore>
__device__ __forceinline__ void valu_partial(const ValuArgs& a, const FusedArgs& f, const int bx, const int h,
                                             const int bz) {
  Lds& sh = g_lds<Store>.v;
  using C = Cfg<D>;
  const int wave = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x) >> 6);
  const int lane = threadIdx.x & 63;
  const int tg = lane / C::LPT, j = lane % C::LPT, j8 = j & 7;
  const int tgv = lane / (D / C::DPL), dl = lane % (D / C::DPL);
  const int P = a.page_size;
  const int tpp = P / kTT;

  // Which sequence and split this workgroup is, and how many splits share
  // the sequence's tiles: the launch grid (split, KV head, sequence) over
  // the plan's tiles, or -- the suffix pass of a batch -- work unit bx
  // of the units shared out by suffix length (bal_share), over the
  // sequence's own tiles.
  int s = bz, sp = bx, base = a.split_base, rem = a.split_rem;
  if constexpr (!FUSED) {
    if (a.bal_units > 0) {
      int n_t, W_t, O_t;
      bal_share(a.seq_lens, a.n_seqs, a.pg_begin * P, a.n_pages_plan * tpp, a.bal_units, lane, n_t, W_t, O_t);
      const int g = bx;
      const unsigned long long hit = __ballot(lane < a.n_seqs && g >= O_t && g < O_t + W_t);
      // a sequence too short to reach past the prefix owns no unit: unit 0
      // reports it (the per-unit length check below covers the others)
      if (g == 0 && h == 0 && threadIdx.x < a.n_seqs) {
        const int Lt = a.seq_lens[threadIdx.x];
        if (Lt - a.q_len < a.pg_begin * P || Lt < a.q_len) set_err(a.d_err, HAD_DERR_SEQLEN);
      }
      if (hit == 0) return;  // a unit left over (uniform over the workgroup)
      s = __builtin_amdgcn_readfirstlane(__ffsll(static_cast<long long>(hit)) - 1);
      sp = g - __builtin_amdgcn_readfirstlane(__shfl(O_t, s));
      const int nsplit = __builtin_amdgcn_readfirstlane(__shfl(W_t, s));
      const int n_tiles = __builtin_amdgcn_readfirstlane(__shfl(n_t, s));
      base = n_tiles / nsplit;
      rem = n_tiles % nsplit;
    }
  }

  // Every global load below is unconditional (addresses clamped to valid
  // memory, results masked afterwards): loads under divergent or uniform
  // branches make the compiler's wait-count bookkeeping fall back to
  // "wait for everything", which would serialise the K/V prefetch.
  //
  // This split owns the tiles [t0, t1) of the plan's tiles (counted from page
  // pg_begin; balanced to within one tile, so no workgroup holds a page more
  // than another), which lie on the pages [pg0, pg1_plan); tiles are numbered
  // from pg0's first token, this split's being [tile_lo, tile_hi).
  const int t0 = sp * base + min(sp, rem);
  const int t1 = t0 + base + (sp < rem ? 1 : 0);
  const int pg0 = a.pg_begin + t0 / tpp;
  const int pg1_plan = a.pg_begin + (t1 + tpp - 1) / tpp;
  const int npg_plan = pg1_plan - pg0;
  const int tile_lo = t0 % tpp, tile_hi = t1 - (t0 / tpp) * tpp;
  const int32_t* pt_row = a.page_table + static_cast<size_t>(s) * a.max_pages;

  // Start-up order.  Vector loads retire in issue order, so the small loads
  // go out first: one page-table entry per thread (a split owns at most
  // kMaxPagesPerSplit = blockDim pages) and one 8-byte piece of the kRows x D
  // query block per thread (loading q per wave instead would send every wave
  // of the GPU to the same few L2 lines at kernel start).  Then the first
  // K/V tile of this wave, whose page id comes from a scalar load, so it is
  // in flight while the small loads are consumed; the second follows just
  // before the workgroup synchronises.
  const int pt_val = pt_row[min(pg0 + static_cast<int>(threadIdx.x), a.max_pages - 1)];
  // fused: wave w owns query row w of the launch (and, in the workgroup that
  // holds the last position, the new token w's key row): raw rows first
  constexpr int E = D / 64;
  const int f_row = min(a.row_base + wave, a.rows - 1);
  const int f_j = f_row / a.G, f_hq = h * a.G + f_row % a.G;
  const int f_t = min(wave, a.q_len - 1);
  RowIn<D> f_qin, f_kin;
  uint16_t f_vraw[E];
  if constexpr (FUSED) {
    row_load<D>(f_qin, f.qg + ((static_cast<size_t>(s) * a.q_len + f_j) * a.H_q + f_hq) * 2 * D, f.w_q, lane);
    const size_t kr = ((static_cast<size_t>(s) * a.q_len + f_t) * a.H_kv + h) * D;
    row_load<D>(f_kin, f.k_new + kr, f.w_k, lane);
#pragma unroll
    for (int m = 0; m < E; ++m) f_vraw[m] = f.v_new[kr + lane + 64 * m];
  }
  constexpr int PER_ROW = D / 4;  // 8-byte q pieces per row
  const int q_r = threadIdx.x / PER_ROW, q_c4 = threadIdx.x % PER_ROW;
  const int q_row = a.row_base + min(q_r, kRows - 1);
  uint2 q_piece = make_uint2(0u, 0u);
  if constexpr (!FUSED)
    q_piece = *reinterpret_cast<const uint2*>(
        a.q + ((static_cast<size_t>(s) * a.q_len + (q_row < a.rows ? q_row : 0) / a.G) * a.H_q + h * a.G +
               (q_row < a.rows ? q_row : 0) % a.G) * D + q_c4 * 4);

  // The first two tiles of this wave.  A tile past the length or the split
  // is loaded for nothing and never used.  Buffer 0 is requested here,
  // buffer 1 just before the setup barrier: the small loads of the setup
  // return behind whatever K/V requests the CUs issued before them, and with
  // one tile per wave in the first burst (16 MB over the chip at head_dim
  // 256) they come back sooner while the burst still keeps HBM busy.
  // (Issue order: all of buffer 0, then all of buffer 1, the order the loop
  // refills them in, so the wait counts inside the loop stay exact.)
  Tile<D> buf[2];
  int tcur[2] = {tile_lo + wave, tile_lo + wave + kWaves};
  // both page ids and the length in one scalar round trip (the fences keep
  // the loads adjacent: left to itself the scheduler waits for the first
  // before it computes the next address; the length, needed for the
  // prologue's angles, would otherwise be a second round trip after the
  // first tile's loads)
  const int pix0 = min(pg0 + tcur[0] / tpp, a.max_pages - 1), pix1 = min(pg0 + tcur[1] / tpp, a.max_pages - 1);
  __builtin_amdgcn_sched_barrier(0);
  int pid0[2] = {pt_row[pix0], pt_row[pix1]};
  const int L = a.seq_lens[s];  // (scalar loads: they do not queue behind the tiles)
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int b = 0; b < 2; ++b) pid0[b] = (pid0[b] < 0 || pid0[b] >= a.num_pages) ? 0 : pid0[b];
  __builtin_amdgcn_sched_barrier(0);
  load_tile_at<D>(buf[0], a, pid0[0], tcur[0] % tpp, tcur[0] < tile_hi, h, tg, j, tgv, dl);
  __builtin_amdgcn_sched_barrier(0);

  // (a suffix pass also needs every query to see the whole prefix before
  // pg_begin; a length past the plan's pages would leave tokens no split reads)
  const bool bad_len = L - a.q_len < a.pg_begin * P || L < a.q_len || L > a.max_pages * P ||
                       L > (a.pg_begin + a.n_pages_plan) * P;
  // fused: the workgroup whose split holds the last position's tile owns the new tokens
  const int last_tile = (L - 1) / kTT - a.pg_begin * tpp;
  const bool own = FUSED && !bad_len && last_tile >= t0 && last_tile < t1;
  int errs = (bad_len && threadIdx.x == 0) ? HAD_DERR_SEQLEN : 0;

  // query block -> LDS (rows past `rows` are zero)
  if constexpr (FUSED) {
    uint16_t* qrow = reinterpret_cast<uint16_t*>(&sh.q[wave][0]);
    float* xrow = &sh.o[wave][0][0];
    if (a.row_base + wave < a.rows) {
      uint16_t y[E];
      row_norm_rope<D>(f_qin, L - a.q_len + f_j, f.R, f.rope_coef, f.eps, xrow, lane, y);
      const size_t orow = ((static_cast<size_t>(s) * a.q_len + f_j) * a.H_q + f_hq) * D;
      const uint16_t* gate = f.qg + ((static_cast<size_t>(s) * a.q_len + f_j) * a.H_q + f_hq) * 2 * D + D;
#pragma unroll
      for (int m = 0; m < E; ++m) {
        qrow[lane + 64 * m] = y[m];
        if (sp == 0) {
          f.gate_out[orow + lane + 64 * m] = gate[lane + 64 * m];
          if (f.q_out) f.q_out[orow + lane + 64 * m] = y[m];
        }
      }
    } else {
#pragma unroll
      for (int m = 0; m < E; ++m) qrow[lane + 64 * m] = 0;
    }
    if (own && wave < a.q_len) {
      // the new token `wave`: normalised, rotated key into the pool and LDS
      const int pos = L - a.q_len + wave;
      uint16_t y[E];
      row_norm_rope<D>(f_kin, pos, f.R, f.rope_coef, f.eps, xrow, lane, y);
      const int pid = pt_row[pos / P];
      const bool ok = pid >= 0 && pid < a.num_pages;
      const size_t dst = ((static_cast<size_t>(ok ? pid : 0) * a.H_kv + h) * P + pos % P) * D;
#pragma unroll
      for (int m = 0; m < E; ++m) {
        sh.knew[wave][lane + 64 * m] = y[m];
        sh.vnew[wave][lane + 64 * m] = f_vraw[m];
        if (ok) {
          f.k_pool[dst + lane + 64 * m] = y[m];
          f.v_pool[dst + lane + 64 * m] = f_vraw[m];
        }
      }
      if (!ok && lane == 0) errs |= HAD_DERR_PAGE;
    }
  } else {
    if (q_r < kRows) sh.q[q_r][q_c4] = (a.row_base + q_r < a.rows) ? q_piece : make_uint2(0u, 0u);
  }
  const int my_row = a.row_base + sigma(j8);

  const int n_pages = bad_len ? 0 : (L + P - 1) / P;
  const int npg = max(min(pg1_plan, n_pages) - pg0, 0);
  const int ntiles = min(npg * tpp, tile_hi);  // end of this split's tiles (tiles past L are masked)
  if (threadIdx.x == 0) {
    sh.next = tile_lo + 2 * kWaves;
    sh.err = 0;
  }
  // checked page ids of the split -> LDS (-1 marks an invalid id)
  if (static_cast<int>(threadIdx.x) < npg_plan) {
    const bool ok = pt_val >= 0 && pt_val < a.num_pages;
    if (!ok && static_cast<int>(threadIdx.x) < npg) errs |= HAD_DERR_PAGE;
    sh.pages[threadIdx.x] = ok ? pt_val : -1;
  }
  // visible-key limit of this lane's QK row (causal inside the draft); when
  // fused the new tokens are left out here and added from LDS at the end
  const int lim = FUSED ? L - a.q_len : (my_row < a.rows) ? (L - a.q_len + my_row / a.G + 1) : L;
  const int lim_min = FUSED ? L - a.q_len : L - a.q_len + 1;  // every row sees positions below this
  const int kv_end = FUSED ? L - a.q_len : L;                   // V rows at or past this are zeroed

  load_tile_at<D>(buf[1], a, pid0[1], tcur[1] % tpp, tcur[1] < tile_hi, h, tg, j, tgv, dl);
  __builtin_amdgcn_sched_barrier(0);
  __syncthreads();

  // q rows in lane order: slot r holds row (r ^ sigma(j8)) of this launch
  uint32_t qr[kRows][C::CH * 4];
#pragma unroll
  for (int r = 0; r < kRows; ++r) {
    const uint4* qrow = reinterpret_cast<const uint4*>(&sh.q[r ^ sigma(j8)][0]);
#pragma unroll
    for (int c = 0; c < C::CH; ++c) {
      const uint4 v = qrow[j + c * C::LPT];
      qr[r][c * 4 + 0] = v.x;
      qr[r][c * 4 + 1] = v.y;
      qr[r][c * 4 + 2] = v.z;
      qr[r][c * 4 + 3] = v.w;
    }
  }

  float o[kRows][C::DPL];
#pragma unroll
  for (int r = 0; r < kRows; ++r)
#pragma unroll
    for (int d = 0; d < C::DPL; ++d) o[r][d] = 0.f;
  float m_run = -INFINITY, l_run = 0.f;

  // Tiles are claimed dynamically: the first two per wave are fixed above,
  // later ones come from an LDS counter, so the two waves sharing a SIMD
  // (which the issue arbiter does not serve equally) finish together.  In
  // deterministic mode wave w takes tiles w + 2*kWaves*i and w + kWaves +
  // 2*kWaves*i (counted from tile_lo) instead.  Claims grow monotonically, so tcur[0] < tcur[1]
  // always: the loop runs while both buffers hold a tile (its only exit test
  // is at the top -- with exits between the two halves the compiler's wait
  // counts at the loop head fall back to waiting for every load), and at
  // most one tile is left for buffer 0 after it.
  auto process = [&](Tile<D>& T, const int tile) __attribute__((always_inline)) {
    const int pg = pg0 + tile / tpp;
    const int pos0 = pg * P + (tile % tpp) * kTT;  // logical position of the tile's token 0
    const bool tile_ok = sh.pages[pg - pg0] >= 0;

    // ---- scores
    float sc[C::TS];
#pragma unroll
    for (int i = 0; i < C::TS; ++i) {
      float acc[kRows];
#pragma unroll
      for (int r = 0; r < kRows; ++r) acc[r] = 0.f;
#pragma unroll
      for (int c = 0; c < C::CH; ++c) {
        const uint32_t kw[4] = {T.k[i][c].x, T.k[i][c].y, T.k[i][c].z, T.k[i][c].w};
#pragma unroll
        for (int w = 0; w < 4; ++w)
#pragma unroll
          for (int r = 0; r < kRows; ++r) acc[r] = dot2_bf16(qr[r][c * 4 + w], kw[w], acc[r]);
      }
#pragma unroll
      for (int r = 0; r < 4; ++r) acc[r] += dpp<DPP_ROW_HALF_MIRROR>(acc[r + 4]);
#pragma unroll
      for (int r = 0; r < 2; ++r) acc[r] += dpp<DPP_QUAD_XOR2>(acc[r + 2]);
      acc[0] += dpp<DPP_QUAD_XOR1>(acc[1]);
      if (C::LPT == 16) acc[0] += dpp<DPP_ROW_ROR8>(acc[0]);
      sc[i] = acc[0] * a.scale_log2;
    }
    const bool masked = !tile_ok || (pos0 + kTT > lim_min);
    if (masked) {
#pragma unroll
      for (int i = 0; i < C::TS; ++i) {
        const int pos = pos0 + i * C::TPS + tg;
        if (!tile_ok || pos >= lim) sc[i] = -INFINITY;
      }
    }

    // ---- online softmax (rows are lane-uniform within groups of LPT)
    float mt = sc[0];
#pragma unroll
    for (int i = 1; i < C::TS; ++i) mt = fmaxf(mt, sc[i]);
    if (C::LPT == 8) mt = fmaxf(mt, dpp<DPP_ROW_ROR8>(mt));
    mt = fmaxf(mt, shfl_xor_f(mt, 16));
    mt = fmaxf(mt, shfl_xor_f(mt, 32));
    const float m_new = fmaxf(m_run, mt);
    const float m_sub = (m_new == -INFINITY) ? 0.f : m_new;
    const float alpha = exp2f(m_run - m_sub);
    float lsum = 0.f;
    uint16_t pb[C::TS];
#pragma unroll
    for (int i = 0; i < C::TS; ++i) {
      pb[i] = f32_to_bf16(exp2f(sc[i] - m_sub));
      lsum += bf16_to_f32(pb[i]);
    }
    l_run = l_run * alpha + lsum;
    m_run = m_new;

    // ---- publish p pairs and alpha to the wave's LDS slice
    if (C::LPT == 8 || j < 8) {
      uint16_t* pw = reinterpret_cast<uint16_t*>(&sh.p[wave][0][0]);
#pragma unroll
      for (int i = 0; i < C::TS; ++i) {
        const int t = i * C::TPS + tg;  // token within the tile
        const int g = t % C::TG, vi = t / C::TG;
        const int pair = (vi >> 1) * C::TG + g, half = vi & 1;
        pw[(pair * kRows + sigma(j8)) * 2 + half] = pb[i];
      }
      if (tg == 0) sh.alpha[wave][sigma(j8)] = alpha;
    }
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");

    // ---- rescale and accumulate P V
    const float4 a0 = *reinterpret_cast<const float4*>(&sh.alpha[wave][0]);
    const float4 a1 = *reinterpret_cast<const float4*>(&sh.alpha[wave][4]);
    const float al[kRows] = {a0.x, a0.y, a0.z, a0.w, a1.x, a1.y, a1.z, a1.w};
    bool need = false;
#pragma unroll
    for (int r = 0; r < kRows; ++r) need |= al[r] != 1.f;
    if (need) {
#pragma unroll
      for (int r = 0; r < kRows; ++r)
#pragma unroll
        for (int d = 0; d < C::DPL; ++d) o[r][d] *= al[r];
    }
    // never multiply stale or unchecked rows: zero V past the length or in
    // an invalid page (selects, not a branch: a branch that rewrites load
    // destinations spoils the compiler's wait counts for the other buffer)
    const int vlim = tile_ok ? kv_end - pos0 : 0;
#pragma unroll
    for (int i = 0; i < C::VPL; ++i) {
      const bool keep = tgv + C::TG * i < vlim;
      T.v[i].x = keep ? T.v[i].x : 0u;
      T.v[i].y = keep ? T.v[i].y : 0u;
    }
#pragma unroll
    for (int k = 0; k < C::NPAIR; ++k) {
      const uint4 p0 = *reinterpret_cast<const uint4*>(&sh.p[wave][k * C::TG + tgv][0]);
      const uint4 p1 = *reinterpret_cast<const uint4*>(&sh.p[wave][k * C::TG + tgv][4]);
      const uint32_t pr[kRows] = {p0.x, p0.y, p0.z, p0.w, p1.x, p1.y, p1.z, p1.w};
      const uint2 va = T.v[2 * k], vb = T.v[2 * k + 1];
      const uint32_t vp[4] = {perm_b32(vb.x, va.x, 0x05040100u), perm_b32(vb.x, va.x, 0x07060302u),
                              perm_b32(vb.y, va.y, 0x05040100u), perm_b32(vb.y, va.y, 0x07060302u)};
#pragma unroll
      for (int r = 0; r < kRows; ++r)
#pragma unroll
        for (int d = 0; d < 4; ++d) o[r][d] = dot2_bf16(pr[r], vp[d], o[r][d]);
    }
    __builtin_amdgcn_wave_barrier();

  };
  auto refill = [&](Tile<D>& T, int& tc) __attribute__((always_inline)) {
    // claim the next tile for this buffer and start its loads; past the end
    // the loads cover no bytes (zeros, never used)
    int nxt = tc + 2 * kWaves;
    if (!a.deterministic) {
      if (lane == 0) nxt = atomicAdd(&sh.next, 1);
      nxt = __builtin_amdgcn_readfirstlane(nxt);
    }
    tc = nxt;
    const int nc = min(nxt, ntiles - 1);
    const int pid = sh.pages[nc / tpp];
    load_tile_at<D>(T, a, pid < 0 ? 0 : pid, nc % tpp, nxt < ntiles, h, tg, j, tgv, dl);
    // keep the refill here: the scheduler would otherwise sink it below the
    // wait for the other buffer, halving the prefetch distance
    __builtin_amdgcn_sched_barrier(0);
  };
  while (tcur[1] < ntiles) {
    process(buf[0], tcur[0]);
    refill(buf[0], tcur[0]);
    process(buf[1], tcur[1]);
    refill(buf[1], tcur[1]);
  }
  if (tcur[0] < ntiles) process(buf[0], tcur[0]);

  // ---- wave totals: l over token groups, o over PV token groups
  if (C::LPT == 8) l_run += dpp<DPP_ROW_ROR8>(l_run);
  l_run += shfl_xor_f(l_run, 16);
  l_run += shfl_xor_f(l_run, 32);
#pragma unroll
  for (int r = 0; r < kRows; ++r)
#pragma unroll
    for (int d = 0; d < C::DPL; ++d) {
      if (C::TG >= 4) o[r][d] += shfl_xor_f(o[r][d], 16);
      if (C::TG >= 2) o[r][d] += shfl_xor_f(o[r][d], 32);
    }
  if (tgv == 0) {
#pragma unroll
    for (int r = 0; r < kRows; ++r)
      *reinterpret_cast<float4*>(&sh.o[wave][r][dl * 4]) = make_float4(o[r][0], o[r][1], o[r][2], o[r][3]);
  }
  if (tg == 0 && j < 8) {
    sh.ml[wave][sigma(j8)][0] = m_run;
    sh.ml[wave][sigma(j8)][1] = l_run;
  }
  if constexpr (FUSED) {
    // the new tokens' contribution (workgroup that owns them): wave w adds
    // them for query row w from the LDS copies, causal inside the draft
    if (own) {
      const int r = wave, row = a.row_base + r;
      float* orow = &sh.o[kWaves][r][0];
      float mx = -INFINITY, lsum = 0.f, acc[E];
#pragma unroll
      for (int e = 0; e < E; ++e) acc[e] = 0.f;
      if (row < a.rows) {
        const int jq = row / a.G;  // this row's query token sees new tokens 0..jq
        const uint16_t* qrow = reinterpret_cast<const uint16_t*>(&sh.q[r][0]);
        float qv[E], sc[kRows];
#pragma unroll
        for (int e = 0; e < E; ++e) qv[e] = bf16_to_f32(qrow[lane + 64 * e]);
#pragma unroll
        for (int t = 0; t < kRows; ++t) {
          float dsum = 0.f;
          if (t <= jq) {
#pragma unroll
            for (int e = 0; e < E; ++e) dsum += qv[e] * bf16_to_f32(sh.knew[t][lane + 64 * e]);
#pragma unroll
            for (int off = 32; off >= 1; off >>= 1) dsum += shfl_xor_f(dsum, off);
          }
          sc[t] = (t <= jq) ? dsum * a.scale_log2 : -INFINITY;
          mx = fmaxf(mx, sc[t]);
        }
#pragma unroll
        for (int t = 0; t < kRows; ++t) {
          if (t <= jq) {
            const float pt = bf16_to_f32(f32_to_bf16(exp2f(sc[t] - mx)));
            lsum += pt;
#pragma unroll
            for (int e = 0; e < E; ++e) acc[e] += pt * bf16_to_f32(sh.vnew[t][lane + 64 * e]);
          }
        }
      }
#pragma unroll
      for (int e = 0; e < E; ++e) orow[lane + 64 * e] = acc[e];
      if (lane == 0) {
        sh.ml[kWaves][r][0] = mx;
        sh.ml[kWaves][r][1] = lsum;
      }
    }
  }
  if (errs) atomicOr(&sh.err, errs);
  __syncthreads();
  if (threadIdx.x == 0 && sh.err) set_err(a.d_err, sh.err);
  const int n_parts = (FUSED && own) ? kWaves + 1 : kWaves;  // partials to merge (uniform)

  // ---- merge the waves and store the split's partial: one float4 of one
  // row per thread, each thread forming its row's wave weights itself (the
  // (m, l) reads are LDS broadcasts), so the merge needs no second barrier
  const size_t unit = (static_cast<size_t>(s) * a.H_kv + h) * a.ns_total + a.split_offset + sp;
  for (int idx = threadIdx.x; idx < kRows * D / 4; idx += blockDim.x) {
    const int r = idx / (D / 4), c4 = idx % (D / 4);
    const int row = a.row_base + r;
    if (row >= a.rows) continue;
    // every LDS read first (part kWaves is read even when absent and then
    // not used), then the arithmetic
    float2 ml[kWaves + 1];
    float4 o4[kWaves + 1];
#pragma unroll
    for (int w = 0; w <= kWaves; ++w) {
      ml[w] = *reinterpret_cast<const float2*>(&sh.ml[w][r][0]);
      o4[w] = *reinterpret_cast<const float4*>(&sh.o[w][r][4 * c4]);
    }
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w <= kWaves; ++w) M = fmaxf(M, w < n_parts ? ml[w].x : -INFINITY);
    const float Ms = (M == -INFINITY) ? 0.f : M;
    float lsum = 0.f;
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
    for (int w = 0; w <= kWaves; ++w) {
      // (v_exp_f32: a weight below 2^-126 flushes to 0)
      const float wt = __builtin_amdgcn_exp2f(ml[w].x - Ms);
      const bool use = w < n_parts;
      lsum += use ? wt * ml[w].y : 0.f;
      acc.x += use ? wt * o4[w].x : 0.f;
      acc.y += use ? wt * o4[w].y : 0.f;
      acc.z += use ? wt * o4[w].z : 0.f;
      acc.w += use ? wt * o4[w].w : 0.f;
    }
    *reinterpret_cast<float4*>(&a.ws_o[(unit * a.ws_rows + row) * D + 4 * c4]) = acc;
    if (c4 == 0) *reinterpret_cast<float2*>(&a.ws_ml[(unit * a.ws_rows + row) * 2]) = make_float2(M, lsum);
  }
}

}  // namespace
}  // namespace had
