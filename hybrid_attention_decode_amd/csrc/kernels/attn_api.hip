// Host entry points of decode_attn: argument checks, split plan, dispatch of
// the partial kernel (VALU below 16 query rows per KV head, MFMA at 16 or
// more) and of the split-K merge.  Split-K over the context keeps every CU
// busy for a single sequence at contexts up to 1M tokens (24-ai.news
// long-context table).
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdint>
#include <mutex>

#include "../host/status.h"
#include "attn_internal.h"
#include "had.h"
#include "prologue_math.h"

using had::fail;

namespace {

constexpr int kTargetUnits = 256;     // one 8-wave workgroup per CU on 256 CUs
constexpr int kMinTilesPerUnit = 32;  // at least 4 tiles of 8 tokens per wave

int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int check_desc(const had_attn_desc* d) {
  if (!d) return fail(HAD_ERR_INVALID_ARG, "decode_attn: desc is NULL");
  if (d->n_seqs < 1 || d->q_len < 1 || d->H_q < 1 || d->H_kv < 1 || d->H_q % d->H_kv != 0)
    return fail(HAD_ERR_INVALID_ARG, "decode_attn: bad head/sequence counts (n_seqs=%d q_len=%d H_q=%d H_kv=%d)",
                d->n_seqs, d->q_len, d->H_q, d->H_kv);
  if (d->head_dim != 64 && d->head_dim != 128 && d->head_dim != 256)
    return fail(HAD_ERR_UNSUPPORTED_SHAPE, "decode_attn: head_dim %d not in {64,128,256}", d->head_dim);
  if (d->page_size < 8 || d->page_size > 256 || d->page_size % 8 != 0)
    return fail(HAD_ERR_UNSUPPORTED_SHAPE, "decode_attn: page_size %d must be a multiple of 8 in [8, 256]",
                d->page_size);
  if (d->num_pages < 1 || d->max_pages < 1)
    return fail(HAD_ERR_INVALID_ARG, "decode_attn: num_pages=%d max_pages=%d", d->num_pages, d->max_pages);
  const int64_t cap = static_cast<int64_t>(d->max_pages) * d->page_size;
  if (d->max_seq_len < 0 || d->max_seq_len > cap)
    return fail(HAD_ERR_INVALID_ARG, "decode_attn: max_seq_len %d outside [0, max_pages*page_size=%lld]",
                d->max_seq_len, static_cast<long long>(cap));
  if (d->num_splits < 0) return fail(HAD_ERR_INVALID_ARG, "decode_attn: num_splits %d < 0", d->num_splits);
  if (d->flags & ~(HAD_ATTN_DETERMINISTIC | HAD_ATTN_GATED_OUTPUT))
    return fail(HAD_ERR_INVALID_ARG, "decode_attn: unknown flags 0x%x", d->flags);
  const int rows = d->q_len * (d->H_q / d->H_kv);
  if (rows > 256) return fail(HAD_ERR_UNSUPPORTED_SHAPE, "decode_attn: %d query rows per KV head > 256", rows);
  return HAD_OK;
}

// The split entry points have no gate to apply at the merge.
int no_gate(const had_attn_desc* d, const char* who) {
  if (d && (d->flags & HAD_ATTN_GATED_OUTPUT))
    return fail(HAD_ERR_INVALID_ARG, "%s: HAD_ATTN_GATED_OUTPUT is not available on this entry point", who);
  return HAD_OK;
}

// Split plan over the pages a sequence can reach (max_seq_len, a host bound,
// so the plan does not depend on device data).  Below 16 rows split i owns
// the tiles [i*b + min(i, r), (i+1)*b + min(i+1, r)) of the N = n * page_size
// / 8 tiles of 8 tokens, b = N / ns, r = N % ns (balanced to within one tile;
// such a range can start and end inside a page, so it touches at most
// ceil(n/ns) + 1 pages, and the plan keeps ceil(n/ns) <= 511 when ns > 1);
// at 16 or more rows the pages [i*n/ns, (i+1)*n/ns) (within one page, at
// most 512), except with pages of a multiple of 32 tokens above 64 rows or
// at head_dim >= 128, where the ranges are of 32-token stages (balanced to
// within one stage, one page more than their share like the tile ranges, so
// again at most 511).
int plan(const had_attn_desc* d, int* ns_out, int* pps_out, int* n_pages_out) {
  const int64_t max_len = d->max_seq_len > 0 ? d->max_seq_len : static_cast<int64_t>(d->max_pages) * d->page_size;
  const int64_t n_pages = std::max<int64_t>(1, ceil_div(max_len, d->page_size));
  const int64_t rows_kv = static_cast<int64_t>(d->q_len) * (d->H_q / d->H_kv);
  // ranges that can straddle one page more than their share: the VALU
  // path's tile ranges, and the 32-token-stage ranges of the MFMA kernel
  // that loads K and V straight into LDS (pages of a multiple of 32 tokens,
  // above 64 rows or at head_dim >= 128)
  const bool straddle =
      rows_kv < 16 || (rows_kv >= 16 && d->page_size % 32 == 0 && (rows_kv > 64 || d->head_dim >= 128));
  int64_t ns;
  if (d->num_splits > 0) {
    ns = d->num_splits;
  } else {
    // one 8-wave workgroup per CU on either path; a VALU unit covers at
    // least 4 tiles of 8 tokens per wave, an MFMA unit (>= 16 rows) at least
    // 4 iterations of 64 tokens
    const bool mfma = rows_kv >= 16;
    const int64_t units = static_cast<int64_t>(d->n_seqs) * d->H_kv;
    const int64_t want = std::max<int64_t>(1, ceil_div(kTargetUnits, units));
    const int64_t min_pps = mfma ? ceil_div(256, d->page_size) : ceil_div(kMinTilesPerUnit, d->page_size / 8);
    ns = std::max<int64_t>(1, std::min<int64_t>(want, n_pages / min_pps));
    if (mfma) {
      // whole-page ranges: as many splits as the shortest longest split
      // needs (q pages), if that is more -- 781 pages: 196 splits of <= 4
      // pages rather than 195 with one of 5
      const int64_t q = std::max<int64_t>(min_pps, ceil_div(n_pages, want));
      ns = std::max<int64_t>(ns, std::min<int64_t>(want, ceil_div(n_pages, q)));
    }
    // (below 16 rows a tile range, above 64 rows with pages of a multiple of
    // 32 tokens a range of 32-token stages, can touch one page more)
    const int64_t cap = straddle ? had::kMaxPagesPerSplit - 1 : had::kMaxPagesPerSplit;
    if (n_pages > had::kMaxPagesPerSplit) ns = std::max<int64_t>(ns, ceil_div(n_pages, cap));
  }
  const int64_t pps = ceil_div(n_pages, ns);
  // the VALU path's tile ranges and the 128-row MFMA path's stage ranges can
  // straddle one page more than their share
  const int64_t pps_max = (ns > 1 && straddle) ? had::kMaxPagesPerSplit - 1 : had::kMaxPagesPerSplit;
  if (pps > pps_max)
    return fail(HAD_ERR_UNSUPPORTED_SHAPE, "decode_attn: %lld splits leave %lld pages per split (max %lld)",
                static_cast<long long>(ns), static_cast<long long>(pps), static_cast<long long>(pps_max));
  if (ns > had::kMaxSplits)
    return fail(HAD_ERR_UNSUPPORTED_SHAPE, "decode_attn: %lld splits (max %d)", static_cast<long long>(ns),
                had::kMaxSplits);
  *ns_out = static_cast<int>(ns);
  *pps_out = static_cast<int>(pps);
  if (n_pages_out) *n_pages_out = static_cast<int>(n_pages);
  return HAD_OK;
}

size_t ws_partials_bytes(const had_attn_desc* d, int ns) {
  const size_t rows = static_cast<size_t>(d->q_len) * (d->H_q / d->H_kv);
  return static_cast<size_t>(d->n_seqs) * d->H_kv * ns * rows * (d->head_dim + 2) * sizeof(float);
}

// partials, then (256-byte aligned) a bf16 q block [n_seqs][q_len][H_q][D]
// that had_decode_attn_layer uses when the prologue runs as its own kernel
size_t ws_q_offset(const had_attn_desc* d, int ns) { return (ws_partials_bytes(d, ns) + 255) & ~size_t(255); }

size_t ws_bytes(const had_attn_desc* d, int ns) {
  return ws_q_offset(d, ns) +
         static_cast<size_t>(d->n_seqs) * d->q_len * d->H_q * d->head_dim * sizeof(uint16_t);
}

// Workspace of had_decode_attn_layer_static: one array per GPU, in the code
// object's device memory (allocated when the library's kernels are loaded on
// a device, held until the process ends).  Host code never uses its name as
// an address: the device address comes from hipGetSymbolAddress, once per
// device, and is kept in scratch_addr.
static __device__ __align__(256) unsigned char scratch[HAD_STATIC_WORKSPACE_BYTES];

constexpr int kMaxDevices = 64;
std::mutex scratch_mu;
void* scratch_addr[kMaxDevices] = {};

int scratch_for_current_device(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(HAD_ERR_HIP, "decode_attn_layer_static: hipGetDevice: %s", hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices)
    return fail(HAD_ERR_HIP, "decode_attn_layer_static: device %d outside [0, %d)", dev, kMaxDevices);
  std::lock_guard<std::mutex> lock(scratch_mu);
  if (!scratch_addr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p)
      return fail(HAD_ERR_HIP, "decode_attn_layer_static: hipGetSymbolAddress on device %d: %s", dev,
                  hipGetErrorString(e));
    scratch_addr[dev] = p;
  }
  *out = scratch_addr[dev];
  return HAD_OK;
}

}  // namespace

extern "C" {

int had_decode_attn_plan(const had_attn_desc* d, int32_t* num_splits, int32_t* pages_per_split) {
  if (!num_splits || !pages_per_split) return fail(HAD_ERR_INVALID_ARG, "decode_attn_plan: NULL output");
  int st = check_desc(d);
  if (st != HAD_OK) return st;
  int ns, pps;
  st = plan(d, &ns, &pps, nullptr);
  if (st != HAD_OK) return st;
  *num_splits = ns;
  *pages_per_split = pps;
  return had::ok();
}

size_t had_decode_attn_workspace_bytes(const had_attn_desc* d) {
  if (check_desc(d) != HAD_OK) return 0;
  int ns, pps;
  if (plan(d, &ns, &pps, nullptr) != HAD_OK) return 0;
  return ws_bytes(d, ns);
}

// fused != nullptr: the prologue runs inside the partial kernel (p->q unused)
static int launch_partial(const had_attn_desc* d, const had_attn_ptrs* p, void* stream, had::ValuArgs* out_args,
                          const had::FusedArgs* fused = nullptr) {
  int st = check_desc(d);
  if (st != HAD_OK) return st;
  if (!p || (!p->q && !fused) || !p->k_pool || !p->v_pool || !p->page_table || !p->seq_lens || !p->workspace)
    return fail(HAD_ERR_INVALID_ARG, "decode_attn: NULL pointer in ptrs");
  if ((!fused && !aligned16(p->q)) || !aligned16(p->k_pool) || !aligned16(p->v_pool) || !aligned16(p->workspace))
    return fail(HAD_ERR_INVALID_ARG, "decode_attn: q, pools and workspace must be 16-byte aligned");
  int ns, pps, n_plan;
  st = plan(d, &ns, &pps, &n_plan);
  if (st != HAD_OK) return st;
  const size_t need = ws_bytes(d, ns);
  if (p->workspace_bytes < need)
    return fail(HAD_ERR_WORKSPACE_TOO_SMALL, "decode_attn: workspace %zu bytes < %zu", p->workspace_bytes, need);

  const int G = d->H_q / d->H_kv;
  const int rows = d->q_len * G;
  had::ValuArgs a{};
  a.q = static_cast<const uint16_t*>(p->q);
  a.k_pool = static_cast<const uint16_t*>(p->k_pool);
  a.v_pool = static_cast<const uint16_t*>(p->v_pool);
  a.page_table = p->page_table;
  a.seq_lens = p->seq_lens;
  a.ws_o = static_cast<float*>(p->workspace);
  a.ws_ml = a.ws_o + static_cast<size_t>(d->n_seqs) * d->H_kv * ns * rows * d->head_dim;
  a.d_err = p->d_err;
  a.n_seqs = d->n_seqs;
  a.q_len = d->q_len;
  a.H_q = d->H_q;
  a.H_kv = d->H_kv;
  a.G = G;
  a.rows = rows;
  a.num_pages = d->num_pages;
  a.page_size = d->page_size;
  a.max_pages = d->max_pages;
  a.num_splits = ns;
  a.pps = pps;
  a.n_pages_plan = n_plan;
  {
    const int64_t n_tiles = static_cast<int64_t>(n_plan) * (d->page_size / 8);
    a.split_base = static_cast<int>(n_tiles / ns);
    a.split_rem = static_cast<int>(n_tiles % ns);
  }
  a.deterministic = (d->flags & HAD_ATTN_DETERMINISTIC) ? 1 : 0;
  a.scale_log2 = d->sm_scale * 1.4426950408889634f;
  a.pg_begin = 0;
  a.split_offset = 0;
  a.ns_total = ns;
  a.ws_rows = rows;
  a.batch_rows = 0;
  a.fixed_len = -1;

  hipStream_t s = static_cast<hipStream_t>(stream);
  const dim3 grid(ns, d->H_kv, d->n_seqs);
  hipError_t e = hipSuccess;
  if (rows >= 16) {
    a.row_base = 0;
    e = fused ? had::launch_attn_mfma128_fused(a, *fused, d->head_dim, grid, s)
              : had::launch_attn_mfma(a, d->head_dim, grid, s);
  } else {
    for (int rb = 0; rb < rows && e == hipSuccess; rb += 8) {
      a.row_base = rb;
      e = fused ? had::launch_attn_valu_fused(a, *fused, d->head_dim, grid, s)
                : had::launch_attn_valu(a, d->head_dim, grid, s);
    }
  }
  if (e != hipSuccess) return fail(HAD_ERR_HIP, "decode_attn: partial kernel launch: %s", hipGetErrorString(e));
  if (out_args) *out_args = a;
  return HAD_OK;
}

int had_decode_attn_partial(const had_attn_desc* d, const had_attn_ptrs* p, void* stream) {
  if (no_gate(d, "decode_attn_partial") != HAD_OK) return HAD_ERR_INVALID_ARG;
  const int st = launch_partial(d, p, stream, nullptr);
  return st == HAD_OK ? had::ok() : st;
}

// gate / gate_hstride: bf16 gate of head (s, j, hq) at gate + ((s*q_len + j)*H_q + hq)*gate_hstride,
// applied when the descriptor asks for the gated output.
static int launch_combine_after(const had_attn_desc* d, const had::ValuArgs& a, void* out, void* stream,
                                const void* gate = nullptr, int gate_hstride = 0, int bal_units = 0,
                                int prefix_splits = 0, int prefix_tiles = 0, int prefix_weight16 = 0,
                                int min_prefix_units = 0) {
  had::CombineArgs c{};
  if (bal_units > 0) {  // a cascade whose suffix units were shared out by length
    c.seq_lens = a.seq_lens;
    c.bal_units = bal_units;
    c.prefix_splits = prefix_splits;
    c.prefix_tiles = prefix_tiles;  // > 0: one-launch cascade, prefix units computed on the device
    c.prefix_weight16 = prefix_weight16;
    c.min_prefix_units = min_prefix_units;
    c.tok_begin = a.pg_begin * a.page_size;
    c.max_tiles = a.n_pages_plan * (a.page_size / 8);
  }
  if (d->flags & HAD_ATTN_GATED_OUTPUT) {
    c.gate = static_cast<const uint16_t*>(gate);
    c.gate_hstride = gate_hstride;
  }
  c.ws_o = a.ws_o;
  c.ws_ml = a.ws_ml;
  c.out = static_cast<uint16_t*>(out);
  c.n_seqs = a.n_seqs;
  c.q_len = a.q_len;
  c.H_q = a.H_q;
  c.H_kv = a.H_kv;
  c.G = a.G;
  c.rows = a.rows;
  c.num_splits = a.num_splits;
  const hipError_t e = had::launch_attn_combine(c, d->head_dim, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(HAD_ERR_HIP, "decode_attn: combine launch: %s", hipGetErrorString(e));
  return had::ok();
}

int had_decode_attn(const had_attn_desc* d, const had_attn_ptrs* p, void* stream) {
  if (p && !p->out) return fail(HAD_ERR_INVALID_ARG, "decode_attn: out is NULL");
  if (d && p && (d->flags & HAD_ATTN_GATED_OUTPUT) && !p->gate)
    return fail(HAD_ERR_INVALID_ARG, "decode_attn: HAD_ATTN_GATED_OUTPUT with a NULL gate");
  had::ValuArgs a{};
  const int st = launch_partial(d, p, stream, &a);
  if (st != HAD_OK) return st;
  return launch_combine_after(d, a, p->out, stream, p->gate, d->head_dim);
}

static int launch_layer_partial(const had_attn_desc* d, const had_qknrg_desc* pd, const had_qknrg_ptrs* pp,
                                void* workspace, size_t workspace_bytes, void* stream, had::ValuArgs* out_args) {
  int st = check_desc(d);
  if (st != HAD_OK) return st;
  if (!pd || !pp) return fail(HAD_ERR_INVALID_ARG, "decode_attn_layer: NULL argument");
  if (pd->n_seqs != d->n_seqs || pd->T != d->q_len || pd->H_q != d->H_q || pd->H_kv != d->H_kv ||
      pd->head_dim != d->head_dim || pd->num_pages != d->num_pages || pd->page_size != d->page_size ||
      pd->max_pages != d->max_pages)
    return fail(HAD_ERR_INVALID_ARG, "decode_attn_layer: prologue and attention descriptors disagree");
  if (d->q_len > 8)
    return fail(HAD_ERR_UNSUPPORTED_SHAPE, "decode_attn_layer: q_len %d > 8 new tokens", d->q_len);
  if (pd->rotary_dim < 0 || pd->rotary_dim > pd->head_dim || pd->rotary_dim % 2 != 0)
    return fail(HAD_ERR_INVALID_ARG, "decode_attn_layer: rotary_dim %d must be even and <= head_dim", pd->rotary_dim);
  if (!(pd->rope_base > 0.0) || !(pd->eps >= 0.f))
    return fail(HAD_ERR_INVALID_ARG, "decode_attn_layer: rope_base must be > 0 and eps >= 0");
  if (!pp->qg || !pp->k || !pp->v || !pp->w_q || !pp->w_k || !pp->page_table || !pp->seq_lens || !pp->k_pool ||
      !pp->v_pool || !pp->gate_out)
    return fail(HAD_ERR_INVALID_ARG, "decode_attn_layer: NULL pointer in prologue ptrs");
  had::FusedArgs f{};
  f.qg = static_cast<const uint16_t*>(pp->qg);
  f.k_new = static_cast<const uint16_t*>(pp->k);
  f.v_new = static_cast<const uint16_t*>(pp->v);
  f.w_q = pp->w_q;
  f.w_k = pp->w_k;
  f.k_pool = static_cast<uint16_t*>(pp->k_pool);
  f.v_pool = static_cast<uint16_t*>(pp->v_pool);
  f.gate_out = static_cast<uint16_t*>(pp->gate_out);
  f.q_out = static_cast<uint16_t*>(pp->q_out);
  f.rope_coef = had::rope_coef(pd->rope_base, pd->rotary_dim);
  f.eps = pd->eps;
  f.R = pd->rotary_dim;
  had_attn_ptrs p{};
  p.q = nullptr;
  p.k_pool = pp->k_pool;
  p.v_pool = pp->v_pool;
  p.page_table = pp->page_table;
  p.seq_lens = pp->seq_lens;
  p.workspace = workspace;
  p.workspace_bytes = workspace_bytes;
  p.out = nullptr;
  p.d_err = pp->d_err;
  const int rows = d->q_len * (d->H_q / d->H_kv);
  if (rows < 16) return launch_partial(d, &p, stream, out_args, &f);
  // 16..128 rows on the MFMA partial that loads K and V straight into LDS
  // (pages of a multiple of 32 tokens, 16..64 rows at head_dim >= 128):
  // the prologue inline as well (rotation partners a whole number of
  // 32-dim k-steps apart in one lane, or 32 dims apart for R = 64; 16-byte
  // rows for the vector loads and stores)
  const int R = pd->rotary_dim;
  if (rows <= 128 && d->page_size % 32 == 0 && (rows > 64 || d->head_dim >= 128) &&
      (R == 0 || R == 64 || R % 128 == 0) && aligned16(pp->qg) && aligned16(pp->w_q) && aligned16(pp->w_k) &&
      aligned16(pp->gate_out) && (!pp->q_out || aligned16(pp->q_out)))
    return launch_partial(d, &p, stream, out_args, &f);
  // other MFMA shapes: the prologue once as its own kernel, q to the
  // caller's q_out or to the workspace's q block
  int ns, pps, n_plan;
  st = plan(d, &ns, &pps, &n_plan);
  if (st != HAD_OK) return st;
  if (workspace_bytes < ws_bytes(d, ns))
    return fail(HAD_ERR_WORKSPACE_TOO_SMALL, "decode_attn_layer: workspace %zu bytes < %zu", workspace_bytes,
                ws_bytes(d, ns));
  had_qknrg_ptrs pq = *pp;
  if (!pq.q_out) pq.q_out = static_cast<char*>(workspace) + ws_q_offset(d, ns);
  // (a sequence past the plan's pages, which the attention skips, gets no
  // K/V row either)
  st = had::launch_qk_norm_rope_gate(pd, &pq, static_cast<int64_t>(n_plan) * d->page_size, stream);
  if (st != HAD_OK) return st;
  p.q = pq.q_out;
  return launch_partial(d, &p, stream, out_args);
}

int had_decode_attn_layer(const had_attn_desc* d, const had_qknrg_desc* pd, const had_qknrg_ptrs* pp, void* workspace,
                          size_t workspace_bytes, void* out, void* stream) {
  if (!out) return fail(HAD_ERR_INVALID_ARG, "decode_attn_layer: out is NULL");
  had::ValuArgs a{};
  int st = launch_layer_partial(d, pd, pp, workspace, workspace_bytes, stream, &a);
  if (st != HAD_OK) return st;
  // the gate half of each head's (q, gate) pair in qg
  st = launch_combine_after(d, a, out, stream, static_cast<const uint16_t*>(pp->qg) + d->head_dim, 2 * d->head_dim);
  return st == HAD_OK ? had::ok() : st;
}

int had_decode_attn_layer_static(const had_attn_desc* d, const had_qknrg_desc* pd, const had_qknrg_ptrs* pp,
                                 void* out, void* stream) {
  if (!out) return fail(HAD_ERR_INVALID_ARG, "decode_attn_layer_static: out is NULL");
  int st = check_desc(d);
  if (st != HAD_OK) return st;
  int ns, pps;
  st = plan(d, &ns, &pps, nullptr);
  if (st != HAD_OK) return st;
  const size_t need = ws_bytes(d, ns);
  if (need > HAD_STATIC_WORKSPACE_BYTES)
    return fail(HAD_ERR_WORKSPACE_TOO_SMALL,
                "decode_attn_layer_static: the layer needs %zu workspace bytes, the static array holds %zu", need,
                static_cast<size_t>(HAD_STATIC_WORKSPACE_BYTES));
  void* ws = nullptr;
  st = scratch_for_current_device(&ws);
  if (st != HAD_OK) return st;
  return had_decode_attn_layer(d, pd, pp, ws, HAD_STATIC_WORKSPACE_BYTES, out, stream);
}

int had_decode_attn_layer_partial(const had_attn_desc* d, const had_qknrg_desc* pd, const had_qknrg_ptrs* pp,
                                  void* workspace, size_t workspace_bytes, void* stream) {
  if (no_gate(d, "decode_attn_layer_partial") != HAD_OK) return HAD_ERR_INVALID_ARG;
  had::ValuArgs a{};
  const int st = launch_layer_partial(d, pd, pp, workspace, workspace_bytes, stream, &a);
  return st == HAD_OK ? had::ok() : st;
}

int had_decode_attn_combine(const had_attn_desc* d, int32_t num_splits, const void* workspace, void* out,
                            void* stream) {
  int st = check_desc(d);
  if (st != HAD_OK) return st;
  if (no_gate(d, "decode_attn_combine") != HAD_OK) return HAD_ERR_INVALID_ARG;
  if (!workspace || !out || num_splits < 1 || num_splits > had::kMaxSplits)
    return fail(HAD_ERR_INVALID_ARG, "decode_attn_combine: bad argument (num_splits=%d, max %d)", num_splits,
                had::kMaxSplits);
  const int G = d->H_q / d->H_kv;
  const int rows = d->q_len * G;
  had::CombineArgs c{};
  c.ws_o = static_cast<const float*>(workspace);
  c.ws_ml = c.ws_o + static_cast<size_t>(d->n_seqs) * d->H_kv * num_splits * rows * d->head_dim;
  c.out = static_cast<uint16_t*>(out);
  c.n_seqs = d->n_seqs;
  c.q_len = d->q_len;
  c.H_q = d->H_q;
  c.H_kv = d->H_kv;
  c.G = G;
  c.rows = rows;
  c.num_splits = num_splits;
  hipError_t e = had::launch_attn_combine(c, d->head_dim, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(HAD_ERR_HIP, "decode_attn_combine: launch: %s", hipGetErrorString(e));
  return had::ok();
}

// ---- shared-prefix (cascade) attention -----------------------------------
// The batch's common prefix (prefix_pages whole pages, the same page ids at
// the start of every sequence's page table) is read once for the query rows
// of every sequence (MFMA kernel, rows of all sequences in one launch set);
// each sequence's suffix is read by the usual kernel from page prefix_pages
// on; both write partials into one workspace (prefix splits first) and the
// ordinary combine merges them.  Same result as had_decode_attn.
// Suffix pass shared out by length (below 16 rows): G work units per KV
// head over all sequences' suffixes, when every unit's tiles fit one split's
// page list and the merge's per-sequence share fits one wave (n_seqs <= 64).
static int cascade_bal_units(const had_attn_desc* d, int n_sfx) {
  const int rows = d->q_len * (d->H_q / d->H_kv);
  if (rows >= 16 || d->n_seqs > 64 || n_sfx > had::kMaxPagesPerSplit - 2 || d->num_splits != 0) return 0;
  return std::max<int>(d->n_seqs, static_cast<int>(ceil_div(kTargetUnits, d->H_kv)));
}

// Units per KV head of the one-launch cascade (both passes in one grid), or 0
// where it does not apply: suffix units shared out by length, at most 8 rows
// per sequence and 128 in the prefix pass (one row block each), pages of a
// multiple of 32 tokens.  At least one unit per sequence plus the prefix's
// minimum (page cap), and no more slots than the two-pass plan's workspace.
static int cascade_one_launch_units(const had_attn_desc* d, const had_attn_prefix* px, int bal, int ns_p, int ns_s) {
  const int rows = d->q_len * (d->H_q / d->H_kv);
  if (bal <= 0 || rows > 8 || d->n_seqs * rows > 128 || d->page_size % 32 != 0) return 0;
  const int min_pu = static_cast<int>(ceil_div(px->prefix_pages, had::kMaxPagesPerSplit - 1));
  const int G = std::max<int>(static_cast<int>(ceil_div(kTargetUnits, d->H_kv)), min_pu + d->n_seqs);
  return G <= ns_p + ns_s ? G : 0;
}

static int cascade_plan(const had_attn_desc* d, const had_attn_prefix* px, int* ns_p, int* ns_s, int* n_sfx,
                        int* bal = nullptr) {
  int st = check_desc(d);
  if (st != HAD_OK) return st;
  if (!px || px->prefix_pages < 1)
    return fail(HAD_ERR_INVALID_ARG, "decode_attn_cascade: prefix_pages must be >= 1");
  const int64_t max_len = d->max_seq_len > 0 ? d->max_seq_len : static_cast<int64_t>(d->max_pages) * d->page_size;
  const int64_t prefix_len = static_cast<int64_t>(px->prefix_pages) * d->page_size;
  if (prefix_len + d->q_len > max_len || px->prefix_pages > d->max_pages)
    return fail(HAD_ERR_INVALID_ARG, "decode_attn_cascade: prefix of %d pages does not fit max_seq_len %lld",
                px->prefix_pages, static_cast<long long>(max_len));
  // prefix pass: one unit per KV head, rows of every sequence (MFMA)
  had_attn_desc dp = *d;
  dp.n_seqs = 1;
  dp.q_len = d->q_len * 16;  // any row count >= 16 selects the MFMA plan
  dp.max_seq_len = static_cast<int32_t>(prefix_len);
  dp.num_splits = 0;
  int pps;
  st = plan(&dp, ns_p, &pps, nullptr);
  if (st != HAD_OK) return st;
  // suffix pass: the usual plan over the pages after the prefix, or units
  // shared out by length (slots for all of them in every sequence's row)
  had_attn_desc ds = *d;
  ds.max_seq_len = static_cast<int32_t>(max_len - prefix_len);
  ds.num_splits = 0;
  st = plan(&ds, ns_s, &pps, n_sfx);
  if (st != HAD_OK) return st;
  const int b = cascade_bal_units(d, *n_sfx);
  if (b > 0) *ns_s = b;
  if (bal) *bal = b;
  if (*ns_p + *ns_s > had::kMaxSplits)
    return fail(HAD_ERR_UNSUPPORTED_SHAPE, "decode_attn_cascade: %d + %d splits (max %d)", *ns_p, *ns_s,
                had::kMaxSplits);
  return HAD_OK;
}

int had_attn_check_prefix(int32_t n_seqs, int32_t max_pages, const int32_t* page_table, int32_t prefix_pages,
                          const int32_t* prefix) {
  if (n_seqs < 0 || max_pages < 1 || prefix_pages < 1 || prefix_pages > max_pages || !prefix ||
      (n_seqs > 0 && !page_table))
    return fail(HAD_ERR_INVALID_ARG, "attn_check_prefix: bad argument (n_seqs=%d max_pages=%d prefix_pages=%d)",
                n_seqs, max_pages, prefix_pages);
  for (int32_t s = 0; s < n_seqs; ++s)
    for (int32_t i = 0; i < prefix_pages; ++i)
      if (page_table[static_cast<size_t>(s) * max_pages + i] != prefix[i])
        return fail(HAD_ERR_INVALID_ARG,
                    "decode_attn_cascade: sequence %d holds page %d at prefix position %d, the prefix list page %d", s,
                    page_table[static_cast<size_t>(s) * max_pages + i], i, prefix[i]);
  return had::ok();
}

size_t had_decode_attn_cascade_workspace_bytes(const had_attn_desc* d, const had_attn_prefix* px) {
  int ns_p, ns_s, n_sfx;
  if (cascade_plan(d, px, &ns_p, &ns_s, &n_sfx) != HAD_OK) return 0;
  return ws_partials_bytes(d, ns_p + ns_s);
}

// passes: 1 = the prefix pass, 2 = the suffix pass, 3 = both; merge = run the combine after them
static int cascade_launch(const had_attn_desc* d, const had_attn_prefix* px, const had_attn_ptrs* p, int passes,
                          bool merge, void* stream, bool one_launch = false) {
  if (merge && d && p && (d->flags & HAD_ATTN_GATED_OUTPUT) && !p->gate)
    return fail(HAD_ERR_INVALID_ARG, "decode_attn_cascade: HAD_ATTN_GATED_OUTPUT with a NULL gate");
  int ns_p, ns_s, n_sfx, bal;
  int st = cascade_plan(d, px, &ns_p, &ns_s, &n_sfx, &bal);
  if (st != HAD_OK) return st;
  if (!p || !p->q || !p->k_pool || !p->v_pool || !p->page_table || !p->seq_lens || !p->workspace ||
      (merge && !p->out) || !px->prefix_page_table)
    return fail(HAD_ERR_INVALID_ARG, "decode_attn_cascade: NULL pointer in ptrs or prefix");
  if (!aligned16(p->q) || !aligned16(p->k_pool) || !aligned16(p->v_pool) || !aligned16(p->workspace))
    return fail(HAD_ERR_INVALID_ARG, "decode_attn_cascade: q, pools and workspace must be 16-byte aligned");
  // both passes in one grid of G1 units per KV head where that applies (the
  // whole call only: the split entry points keep the two-pass layout, which
  // their merge expects), its G1 slots inside the two-pass workspace
  const int G1 = one_launch ? cascade_one_launch_units(d, px, bal, ns_p, ns_s) : 0;
  const int ns_total = G1 > 0 ? G1 : ns_p + ns_s;
  const size_t need = ws_partials_bytes(d, ns_p + ns_s);
  if (p->workspace_bytes < need)
    return fail(HAD_ERR_WORKSPACE_TOO_SMALL, "decode_attn_cascade: workspace %zu bytes < %zu", p->workspace_bytes,
                need);
  const int G = d->H_q / d->H_kv;
  const int rows = d->q_len * G;
  hipStream_t s = static_cast<hipStream_t>(stream);
  had::ValuArgs a{};
  a.q = static_cast<const uint16_t*>(p->q);
  a.k_pool = static_cast<const uint16_t*>(p->k_pool);
  a.v_pool = static_cast<const uint16_t*>(p->v_pool);
  a.ws_o = static_cast<float*>(p->workspace);
  a.ws_ml = a.ws_o + static_cast<size_t>(d->n_seqs) * d->H_kv * ns_total * rows * d->head_dim;
  a.d_err = p->d_err;
  a.q_len = d->q_len;
  a.H_q = d->H_q;
  a.H_kv = d->H_kv;
  a.G = G;
  a.num_pages = d->num_pages;
  a.page_size = d->page_size;
  a.deterministic = (d->flags & HAD_ATTN_DETERMINISTIC) ? 1 : 0;
  a.scale_log2 = d->sm_scale * 1.4426950408889634f;
  a.ns_total = ns_total;
  a.ws_rows = rows;
  // prefix pass: all sequences' rows, the prefix page list as page-table row 0
  had::ValuArgs ap = a;
  ap.page_table = px->prefix_page_table;
  ap.seq_lens = p->seq_lens;  // unused (fixed_len)
  ap.n_seqs = 1;
  ap.rows = d->n_seqs * rows;
  ap.max_pages = px->prefix_pages;
  ap.num_splits = ns_p;
  ap.pps = 0;
  ap.n_pages_plan = px->prefix_pages;
  ap.pg_begin = 0;
  ap.split_offset = 0;
  ap.batch_rows = rows;
  ap.fixed_len = px->prefix_pages * d->page_size;
  // suffix pass: each sequence from page prefix_pages on
  had::ValuArgs as = a;
  as.page_table = p->page_table;
  as.seq_lens = p->seq_lens;
  as.n_seqs = d->n_seqs;
  as.rows = rows;
  as.max_pages = d->max_pages;
  as.num_splits = ns_s;
  as.pps = 0;
  as.n_pages_plan = n_sfx;
  {
    const int64_t n_tiles = static_cast<int64_t>(n_sfx) * (d->page_size / 8);
    as.split_base = static_cast<int>(n_tiles / ns_s);
    as.split_rem = static_cast<int>(n_tiles % ns_s);
  }
  as.pg_begin = px->prefix_pages;
  as.split_offset = ns_p;
  as.batch_rows = 0;
  as.fixed_len = -1;
  as.bal_units = bal;
  const int prefix_tiles = px->prefix_pages * (d->page_size / 8);
  const int weight16 = had::cascade_prefix_weight16(d->n_seqs * rows);
  const int min_pu = static_cast<int>(ceil_div(px->prefix_pages, had::kMaxPagesPerSplit - 1));
  hipError_t e = hipSuccess;
  if (G1 > 0) {
    if (passes == 3) {
      had::ValuArgs as1 = as;
      as1.bal_units = 0;  // set per workgroup
      as1.row_base = 0;
      ap.row_base = 0;
      e = had::launch_attn_cascade(ap, as1, prefix_tiles, weight16, min_pu, d->head_dim, dim3(G1, d->H_kv, 1), s);
      if (e != hipSuccess)
        return fail(HAD_ERR_HIP, "decode_attn_cascade: one-launch kernel: %s", hipGetErrorString(e));
    }
  } else {
    if (passes & 1) {
      e = had::launch_attn_mfma(ap, d->head_dim, dim3(ns_p, d->H_kv, 1), s);
      if (e != hipSuccess)
        return fail(HAD_ERR_HIP, "decode_attn_cascade: prefix kernel launch: %s", hipGetErrorString(e));
    }
    if (passes & 2) {
      const dim3 grid(ns_s, d->H_kv, bal > 0 ? 1 : d->n_seqs);
      if (rows >= 16) {
        as.row_base = 0;
        e = had::launch_attn_mfma(as, d->head_dim, grid, s);
      } else {
        for (int rb = 0; rb < rows && e == hipSuccess; rb += 8) {
          as.row_base = rb;
          e = had::launch_attn_valu(as, d->head_dim, grid, s);
        }
      }
      if (e != hipSuccess)
        return fail(HAD_ERR_HIP, "decode_attn_cascade: suffix kernel launch: %s", hipGetErrorString(e));
    }
  }
  if (!merge) return had::ok();
  had::ValuArgs am = as;
  am.num_splits = ns_total;
  if (G1 > 0)
    return launch_combine_after(d, am, p->out, stream, p->gate, d->head_dim, G1, 0, prefix_tiles, weight16, min_pu);
  return launch_combine_after(d, am, p->out, stream, p->gate, d->head_dim, bal, ns_p);
}

int had_decode_attn_cascade(const had_attn_desc* d, const had_attn_prefix* px, const had_attn_ptrs* p, void* stream) {
  return cascade_launch(d, px, p, 3, true, stream, true);
}

int had_decode_attn_cascade_plan(const had_attn_desc* d, const had_attn_prefix* px, int32_t* prefix_splits,
                                 int32_t* suffix_splits) {
  if (!prefix_splits || !suffix_splits) return fail(HAD_ERR_INVALID_ARG, "decode_attn_cascade_plan: NULL output");
  int ns_p, ns_s, n_sfx;
  const int st = cascade_plan(d, px, &ns_p, &ns_s, &n_sfx);
  if (st != HAD_OK) return st;
  *prefix_splits = ns_p;
  *suffix_splits = ns_s;
  return had::ok();
}

int had_decode_attn_cascade_partial(const had_attn_desc* d, const had_attn_prefix* px, const had_attn_ptrs* p,
                                    int32_t passes, void* stream) {
  if (no_gate(d, "decode_attn_cascade_partial") != HAD_OK) return HAD_ERR_INVALID_ARG;
  if (passes < 1 || passes > 3)
    return fail(HAD_ERR_INVALID_ARG, "decode_attn_cascade_partial: passes %d not in {1, 2, 3}", passes);
  return cascade_launch(d, px, p, passes, false, stream);
}

int had_decode_attn_cascade_combine(const had_attn_desc* d, const had_attn_prefix* px, const had_attn_ptrs* p,
                                    void* stream) {
  return cascade_launch(d, px, p, 0, true, stream);
}

}  // extern "C"
