// Host entry points of decode_attn: argument checks, split plan, dispatch of
// the partial kernel (VALU below 16 query rows per KV head, MFMA at 16 or
// more) and of the split-K merge.  Split-K over the context keeps every CU
// busy for a single sequence at contexts up to 1M tokens (24-ai.news
// long-context table).
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdint>

#include "../host/status.h"
#include "attn_internal.h"
#include "had.h"

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
  if (d->flags & ~HAD_ATTN_DETERMINISTIC) return fail(HAD_ERR_INVALID_ARG, "decode_attn: unknown flags 0x%x", d->flags);
  const int rows = d->q_len * (d->H_q / d->H_kv);
  if (rows > 256) return fail(HAD_ERR_UNSUPPORTED_SHAPE, "decode_attn: %d query rows per KV head > 256", rows);
  return HAD_OK;
}

// Split plan over the pages a sequence can reach (max_seq_len, a host bound,
// so the plan does not depend on device data).  Split i owns pages
// [i*n/ns, (i+1)*n/ns): balanced to within one page.
int plan(const had_attn_desc* d, int* ns_out, int* pps_out, int* n_pages_out) {
  const int64_t max_len = d->max_seq_len > 0 ? d->max_seq_len : static_cast<int64_t>(d->max_pages) * d->page_size;
  const int64_t n_pages = std::max<int64_t>(1, ceil_div(max_len, d->page_size));
  int64_t ns;
  if (d->num_splits > 0) {
    ns = d->num_splits;
  } else {
    // one 8-wave workgroup per CU on either path; a VALU unit covers at
    // least 4 tiles of 8 tokens per wave, an MFMA unit (>= 16 rows) at least
    // 4 iterations of 64 tokens
    const bool mfma = d->q_len * (d->H_q / d->H_kv) >= 16;
    const int64_t units = static_cast<int64_t>(d->n_seqs) * d->H_kv;
    const int64_t want = std::max<int64_t>(1, ceil_div(kTargetUnits, units));
    const int64_t min_pps = mfma ? ceil_div(256, d->page_size) : ceil_div(kMinTilesPerUnit, d->page_size / 8);
    ns = std::max<int64_t>(1, std::min<int64_t>(want, n_pages / min_pps));
    ns = std::max<int64_t>(ns, ceil_div(n_pages, had::kMaxPagesPerSplit));
  }
  const int64_t pps = ceil_div(n_pages, ns);
  if (pps > had::kMaxPagesPerSplit)
    return fail(HAD_ERR_UNSUPPORTED_SHAPE, "decode_attn: %lld splits leave %lld pages per split (max %d)",
                static_cast<long long>(ns), static_cast<long long>(pps), had::kMaxPagesPerSplit);
  if (ns > had::kMaxSplits)
    return fail(HAD_ERR_UNSUPPORTED_SHAPE, "decode_attn: %lld splits (max %d)", static_cast<long long>(ns),
                had::kMaxSplits);
  *ns_out = static_cast<int>(ns);
  *pps_out = static_cast<int>(pps);
  if (n_pages_out) *n_pages_out = static_cast<int>(n_pages);
  return HAD_OK;
}

size_t ws_bytes(const had_attn_desc* d, int ns) {
  const size_t rows = static_cast<size_t>(d->q_len) * (d->H_q / d->H_kv);
  return static_cast<size_t>(d->n_seqs) * d->H_kv * ns * rows * (d->head_dim + 2) * sizeof(float);
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

static int launch_partial(const had_attn_desc* d, const had_attn_ptrs* p, void* stream, had::ValuArgs* out_args) {
  int st = check_desc(d);
  if (st != HAD_OK) return st;
  if (!p || !p->q || !p->k_pool || !p->v_pool || !p->page_table || !p->seq_lens || !p->workspace)
    return fail(HAD_ERR_INVALID_ARG, "decode_attn: NULL pointer in ptrs");
  if (!aligned16(p->q) || !aligned16(p->k_pool) || !aligned16(p->v_pool) || !aligned16(p->workspace))
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
  a.deterministic = (d->flags & HAD_ATTN_DETERMINISTIC) ? 1 : 0;
  a.scale_log2 = d->sm_scale * 1.4426950408889634f;

  hipStream_t s = static_cast<hipStream_t>(stream);
  const dim3 grid(ns, d->H_kv, d->n_seqs);
  hipError_t e = hipSuccess;
  if (rows >= 16) {
    a.row_base = 0;
    e = had::launch_attn_mfma(a, d->head_dim, grid, s);
  } else {
    for (int rb = 0; rb < rows && e == hipSuccess; rb += 8) {
      a.row_base = rb;
      e = had::launch_attn_valu(a, d->head_dim, grid, s);
    }
  }
  if (e != hipSuccess) return fail(HAD_ERR_HIP, "decode_attn: partial kernel launch: %s", hipGetErrorString(e));
  if (out_args) *out_args = a;
  return HAD_OK;
}

int had_decode_attn_partial(const had_attn_desc* d, const had_attn_ptrs* p, void* stream) {
  const int st = launch_partial(d, p, stream, nullptr);
  return st == HAD_OK ? had::ok() : st;
}

int had_decode_attn(const had_attn_desc* d, const had_attn_ptrs* p, void* stream) {
  if (p && !p->out) return fail(HAD_ERR_INVALID_ARG, "decode_attn: out is NULL");
  had::ValuArgs a{};
  int st = launch_partial(d, p, stream, &a);
  if (st != HAD_OK) return st;
  had::CombineArgs c{};
  c.ws_o = a.ws_o;
  c.ws_ml = a.ws_ml;
  c.out = static_cast<uint16_t*>(p->out);
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

int had_decode_attn_combine(const had_attn_desc* d, int32_t num_splits, const void* workspace, void* out,
                            void* stream) {
  int st = check_desc(d);
  if (st != HAD_OK) return st;
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

}  // extern "C"
