// Device helpers of the paged KV cache: raw append of new K/V rows at their
// page slots, and whole-page copies (the device half of copy-on-write).
//
// Pools are bf16 [num_pages][H_kv][page_size][head_dim]; logical position p
// of sequence s lives in page page_table[s][p / page_size], row
// p % page_size (zubnet.ai TokenSpeed article, second paragraph: KV pages,
// cached checkpoints reused without mutation by copy-on-write).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>

#include "../host/status.h"
#include "had.h"
#include "kcommon.h"

using had::fail;

namespace had {
namespace {

// One block per (sequence, new token); threads copy 16-byte chunks of every
// head's K and V row.
__global__ __launch_bounds__(256) void kv_append_kernel(uint4* k_pool, uint4* v_pool, const int32_t* page_table,
                                                        int max_pages, const int32_t* seq_lens, const uint4* k_new,
                                                        const uint4* v_new, int t_new, int num_pages, int H_kv,
                                                        int P, int D, int32_t* d_err) {
  const int s = blockIdx.x / t_new, j = blockIdx.x % t_new;
  const int L = seq_lens[s];
  const int pos = L - t_new + j;
  if (L < t_new || pos >= max_pages * P) {
    if (threadIdx.x == 0) set_err(d_err, HAD_DERR_SEQLEN);
    return;
  }
  const int pid = page_table[static_cast<size_t>(s) * max_pages + pos / P];
  if (pid < 0 || pid >= num_pages) {
    if (threadIdx.x == 0) set_err(d_err, HAD_DERR_PAGE);
    return;
  }
  const int cpr = D / 8;  // 16-byte chunks per row
  const size_t src_row = (static_cast<size_t>(s) * t_new + j) * H_kv;
  for (int c = threadIdx.x; c < H_kv * cpr; c += blockDim.x) {
    const int h = c / cpr, q = c % cpr;
    const size_t dst = ((static_cast<size_t>(pid) * H_kv + h) * P + pos % P) * cpr + q;
    // both loads before either store (in program order the store to k_pool
    // could alias v_new, so each load would wait for the store before it)
    const uint4 kx = k_new[(src_row + h) * cpr + q], vx = v_new[(src_row + h) * cpr + q];
    k_pool[dst] = kx;
    v_pool[dst] = vx;
  }
}

// blockIdx.y = pair index; blocks along x stride over the page's chunks.
// The pairs live in device memory, so a captured graph can be replayed with
// new pairs; a pair whose source is -1 is an unused entry.  Every block checks
// its own pair before it touches a byte: ids in range (HAD_DERR_PAGE), and
// its destination neither the source of an active pair nor the destination
// of an earlier one (HAD_DERR_COPY) -- two such blocks would race on a page.
// A pair that fails is skipped.
__global__ __launch_bounds__(256) void kv_copy_kernel(uint4* k_pool, uint4* v_pool, const int32_t* d_src,
                                                      const int32_t* d_dst, int n, int num_pages, size_t chunks,
                                                      int32_t* d_err) {
  const int i = blockIdx.y;
  const int src = d_src[i], dst = d_dst[i];
  if (src == -1) return;  // unused entry (uniform over the block)
  if (src < 0 || src >= num_pages || dst < 0 || dst >= num_pages) {
    if (threadIdx.x == 0 && blockIdx.x == 0) set_err(d_err, HAD_DERR_PAGE);
    return;
  }
  int clash = 0;
  for (int k = threadIdx.x; k < n; k += blockDim.x) {
    const int sk = d_src[k];
    if (sk != -1 && (dst == sk || (k < i && dst == d_dst[k]))) clash = 1;
  }
  if (__syncthreads_or(clash)) {
    if (threadIdx.x == 0 && blockIdx.x == 0) set_err(d_err, HAD_DERR_COPY);
    return;
  }
  const size_t so = static_cast<size_t>(src) * chunks, dof = static_cast<size_t>(dst) * chunks;
  for (size_t c = blockIdx.x * blockDim.x + threadIdx.x; c < chunks; c += static_cast<size_t>(gridDim.x) * blockDim.x) {
    // both loads first (source and destination pages differ, so the loads
    // never see either store)
    const uint4 kx = k_pool[so + c], vx = v_pool[so + c];
    k_pool[dof + c] = kx;
    v_pool[dof + c] = vx;
  }
}

int check_layout(const had_kv_layout* L, const char* who) {
  if (!L) return fail(HAD_ERR_INVALID_ARG, "%s: layout is NULL", who);
  if (L->num_pages < 1 || L->H_kv < 1 || L->page_size < 1)
    return fail(HAD_ERR_INVALID_ARG, "%s: bad layout (num_pages=%d H_kv=%d page_size=%d)", who, L->num_pages,
                L->H_kv, L->page_size);
  if (L->head_dim < 8 || L->head_dim % 8 != 0)
    return fail(HAD_ERR_UNSUPPORTED_SHAPE, "%s: head_dim %d must be a positive multiple of 8", who, L->head_dim);
  return HAD_OK;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

}  // namespace
}  // namespace had

extern "C" {

int had_kv_copy_pages(const had_kv_layout* L, void* k_pool, void* v_pool, const int32_t* d_src,
                      const int32_t* d_dst, int32_t n, int32_t* d_err, void* stream) {
  int st = had::check_layout(L, "kv_copy_pages");
  if (st != HAD_OK) return st;
  if (n < 0 || n > 65535 || (n > 0 && (!d_src || !d_dst || !k_pool || !v_pool)))
    return fail(HAD_ERR_INVALID_ARG, "kv_copy_pages: bad argument (n=%d, at most 65535 pairs)", n);
  if (!had::aligned16(k_pool) || !had::aligned16(v_pool))
    return fail(HAD_ERR_INVALID_ARG, "kv_copy_pages: pools must be 16-byte aligned");
  if (n == 0) return had::ok();
  const size_t chunks = static_cast<size_t>(L->H_kv) * L->page_size * L->head_dim / 8;
  const size_t blocks_x = std::min<size_t>(64, (chunks + 255) / 256);
  hipLaunchKernelGGL(had::kv_copy_kernel, dim3(static_cast<unsigned>(blocks_x), n), dim3(256), 0,
                     static_cast<hipStream_t>(stream), static_cast<uint4*>(k_pool), static_cast<uint4*>(v_pool), d_src,
                     d_dst, n, L->num_pages, chunks, d_err);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(HAD_ERR_HIP, "kv_copy_pages: launch: %s", hipGetErrorString(e));
  return had::ok();
}

int had_kv_check_copy_pages(int32_t num_pages, const int32_t* src, const int32_t* dst, int32_t n) {
  if (num_pages < 1 || n < 0 || (n > 0 && (!src || !dst)))
    return fail(HAD_ERR_INVALID_ARG, "kv_check_copy_pages: bad argument (num_pages=%d n=%d)", num_pages, n);
  for (int32_t i = 0; i < n; ++i) {
    if (src[i] == -1) continue;
    if (src[i] < 0 || src[i] >= num_pages || dst[i] < 0 || dst[i] >= num_pages)
      return fail(HAD_ERR_INVALID_ARG, "kv_copy_pages: pair %d (%d -> %d) outside [0, %d)", i, src[i], dst[i],
                  num_pages);
    for (int32_t k = 0; k < n; ++k) {
      if (src[k] == -1) continue;
      if (dst[i] == src[k])
        return fail(HAD_ERR_INVALID_ARG, "kv_copy_pages: page %d is both a source and a destination", dst[i]);
      if (k < i && dst[i] == dst[k])
        return fail(HAD_ERR_INVALID_ARG, "kv_copy_pages: destination %d repeated", dst[i]);
    }
  }
  return had::ok();
}

int had_kv_append(const had_kv_layout* L, void* k_pool, void* v_pool, const int32_t* d_page_table, int32_t max_pages,
                  const int32_t* d_seq_lens, const void* k_new, const void* v_new, int32_t n_seqs, int32_t t_new,
                  int32_t* d_err, void* stream) {
  int st = had::check_layout(L, "kv_append");
  if (st != HAD_OK) return st;
  if (!k_pool || !v_pool || !d_page_table || !d_seq_lens || !k_new || !v_new || n_seqs < 0 || t_new < 0 ||
      max_pages < 1)
    return fail(HAD_ERR_INVALID_ARG, "kv_append: bad argument");
  if (!had::aligned16(k_pool) || !had::aligned16(v_pool) || !had::aligned16(k_new) || !had::aligned16(v_new))
    return fail(HAD_ERR_INVALID_ARG, "kv_append: pools and new rows must be 16-byte aligned");
  if (n_seqs == 0 || t_new == 0) return had::ok();
  hipLaunchKernelGGL(had::kv_append_kernel, dim3(n_seqs * t_new), dim3(256), 0, static_cast<hipStream_t>(stream),
                     static_cast<uint4*>(k_pool), static_cast<uint4*>(v_pool), d_page_table, max_pages, d_seq_lens,
                     static_cast<const uint4*>(k_new), static_cast<const uint4*>(v_new), t_new, L->num_pages,
                     L->H_kv, L->page_size, L->head_dim, d_err);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(HAD_ERR_HIP, "kv_append: launch: %s", hipGetErrorString(e));
  return had::ok();
}

}  // extern "C"
