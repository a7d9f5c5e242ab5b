/*
 * had.h -- C ABI of the hybrid-attention decode library (libhad.so), gfx950.
 *
 * One decode step of a hybrid model (full-attention layers interleaved with
 * Gated DeltaNet layers) as these groups of calls:
 *
 *   kv_page_table      host page-table / state-slot manager, speculative
 *                      rollback, the hybrid prefix cache (radix tree), and
 *                      two device helpers that move KV rows (append,
 *                      copy-on-write copy)
 *   qk_norm_rope_gate  fused prologue of a full-attention layer
 *   decode_attn        split-K GQA decode attention over the paged KV cache
 *                      (plus the shared-prefix "cascade" form and the layer
 *                      entry point with the prologue fused in)
 *   gdn_state_update   gated delta rule update of slot-addressed states
 *   gdn_prefill        the same recurrence over whole prompts, chunk-parallel
 *
 * Sources.  The system is the TokenSpeed inference engine described in a few
 * news articles: zubnet.ai (Spanish/French), second paragraph -- paged KV,
 * Mamba/GDN state slots checkpointed next to the KV, index indirection
 * through current_input_indices instead of tensor copies, copy-on-write reuse
 * of cached checkpoints, the fused QK-RMSNorm + partial RoPE + gate split;
 * 24-ai.news -- the hybrid full-attention / Gated DeltaNet model, the
 * "Mamba State Update" optimisation (O(1) pointer update), hybrid prefix
 * caching with a C++ logical cache over Python-owned physical tensors, and
 * the 128K / 256K / 1M long-context table; evermx.com, "Pluggable Kernel
 * Registry" -- one portable entry point per kernel.  The articles give no
 * formulas; each call below states the operation it computes.
 *
 * Conventions (all calls)
 * -----------------------
 * - Every call returns an int status: HAD_OK (0) or a negative HAD_ERR_*.
 *   Nothing is thrown across the ABI.  had_last_error() returns a
 *   thread-local message describing the last failure on the calling thread.
 * - A failing host call leaves every handle exactly as it was.
 * - The library never allocates device memory.  The caller owns every device
 *   buffer (inputs, outputs, pools, workspaces) and every host handle it
 *   creates.  Device pointers are plain addresses from the caller's
 *   allocator (e.g. torch); "stream" is a hipStream_t passed as void*
 *   (NULL = the default stream).  Device calls only enqueue work on that
 *   stream: no hidden synchronisation, no host<->device copies.
 * - bf16 tensors are IEEE bfloat16 bit patterns; all tensors are dense,
 *   row-major, in the layout written next to each argument.
 * - Alignment (the kernels load 8 or 16 bytes per lane): KV pools, q of the
 *   attention calls, the new K/V rows of had_kv_append, every workspace, the
 *   GDN state pools and the prefill's q, k, v must be 16-byte aligned, the
 *   q and k of had_gdn_state_update 8-byte aligned; a misaligned pointer is
 *   HAD_ERR_INVALID_ARG.  Allocator bases (hipMalloc, torch) always are;
 *   only offset views can violate it.
 * - Device-side index checks: every kernel checks page ids against
 *   num_pages and slot ids against n_slots and skips (never dereferences) an
 *   out-of-range id.  If the optional d_err pointer (device int32) is not
 *   NULL the kernel ORs a HAD_DERR_* bit into it; the caller reads it when
 *   convenient (no device->host round trip is forced).
 */
#ifndef HAD_H
#define HAD_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define HAD_ABI_VERSION 5

enum {
  HAD_OK = 0,
  HAD_ERR_INVALID_ARG = -1,       /* null pointer, negative size, bad value      */
  HAD_ERR_UNSUPPORTED_SHAPE = -2, /* shape outside what the kernels implement    */
  HAD_ERR_OUT_OF_PAGES = -3,      /* free list cannot satisfy a reservation      */
  HAD_ERR_OUT_OF_SLOTS = -4,      /* no free state slot                          */
  HAD_ERR_BAD_SEQ = -5,           /* unknown or freed sequence id                */
  HAD_ERR_WORKSPACE_TOO_SMALL = -6,
  HAD_ERR_HIP = -7,               /* a HIP runtime call failed                   */
  HAD_ERR_BAD_SLOT = -8,          /* slot id out of range or not held            */
  HAD_ERR_CAPACITY = -9,          /* max_seqs or max_pages_per_seq exceeded      */
  HAD_ERR_RANGE = -10             /* length argument outside [0, current length] */
};

/* bits ORed into *d_err by kernels */
enum {
  HAD_DERR_PAGE = 1,    /* page id < 0 or >= num_pages for a position < seq_len */
  HAD_DERR_SLOT = 2,    /* slot id >= n_slots, or out slot < 0                 */
  HAD_DERR_SEQLEN = 4,  /* seq_len < q_len (or T), beyond max_pages*page_size,
                           or (attention) beyond the pages the split plan covers */
  HAD_DERR_COPY = 8     /* page-copy list: a destination that is also a source or
                           repeats an earlier destination                      */
};

int had_abi_version(void);
const char *had_last_error(void);

/* ======================================================================
 * kv_page_table -- host side (C++; no GPU needed)
 *
 * Logical position p of sequence s lives in physical page
 * page_table[s][p / page_size], row p % page_size.  Forked sequences alias
 * the pages of their prefix (reference counts); the first write into a
 * shared, partially filled last page copies it first (copy-on-write).  This
 * is the engine's "logical cache in C++, physical tensors in Python" split
 * (24-ai.news, optimisation list, hybrid prefix caching; zubnet.ai ¶2,
 * copy-on-write of cached checkpoints).
 *
 * Allocation policy (deterministic, so results can be compared bit for bit):
 * the free list starts as `free_order` (identity if NULL); allocation pops
 * its LAST element; a page whose reference count drops to 0 is pushed at the
 * end.  New sequence ids are the lowest unused id.
 * ====================================================================== */
typedef struct had_kvpt had_kvpt;

/* num_pages physical pages of page_size tokens; up to max_seqs live
 * sequences of up to max_pages_per_seq pages each.  free_order: host array
 * of num_pages distinct ids in [0, num_pages) or NULL.  *out receives the
 * handle (owned by the caller; release with had_kvpt_destroy). */
int had_kvpt_create(int32_t num_pages, int32_t page_size, int32_t max_seqs,
                    int32_t max_pages_per_seq, const int32_t *free_order,
                    had_kvpt **out);
int had_kvpt_destroy(had_kvpt *h);

/* New empty sequence; *seq receives its id.  HAD_ERR_CAPACITY when
 * max_seqs sequences are live. */
int had_kvpt_seq_create(had_kvpt *h, int32_t *seq);

/* New sequence sharing the first prefix_len tokens of src: it aliases the
 * first ceil(prefix_len / page_size) pages (each gains a reference).
 * HAD_ERR_RANGE if prefix_len > length of src. */
int had_kvpt_seq_fork(had_kvpt *h, int32_t src, int32_t prefix_len, int32_t *seq);

/* New sequence of length len aliasing the given held pages (each gains a
 * reference): how a request starts from a cached prefix (had_radix_match).
 * HAD_ERR_RANGE unless n_pages == ceil(len / page_size); HAD_ERR_INVALID_ARG
 * if a page is out of range or has no reference.  pages: host int32[n_pages]. */
int had_kvpt_seq_create_from(had_kvpt *h, const int32_t *pages, int32_t n_pages, int32_t len, int32_t *seq);

/* One more / one less reference on a held page (a holder outside any
 * sequence, such as the prefix cache).  HAD_ERR_INVALID_ARG if the page is
 * out of range or has no reference; at 0 the page returns to the free list. */
int had_kvpt_page_retain(had_kvpt *h, int32_t page);
int had_kvpt_page_release(had_kvpt *h, int32_t page);

/* Grow seq by n_tokens (>= 0).  If the last page is partially filled and
 * shared it is first replaced by a fresh page; the copy the caller must then
 * perform on every layer's pools is reported as cow = {src, dst, valid}
 * (valid = tokens already in the page) with *n_cow = 1, else *n_cow = 0.
 * Then fresh pages are appended until the sequence covers its new length.
 * Transactional: HAD_ERR_CAPACITY / HAD_ERR_OUT_OF_PAGES change nothing.
 * cow: host int32[3]; n_cow: host int32. */
int had_kvpt_reserve(had_kvpt *h, int32_t seq, int32_t n_tokens, int32_t *cow,
                     int32_t *n_cow);

/* Shrink seq to new_len (<= length): pages past ceil(new_len / page_size)
 * are dropped, last first; a page that loses its last reference goes back to
 * the free list.  Stale rows left in a kept page are masked by the length. */
int had_kvpt_truncate(had_kvpt *h, int32_t seq, int32_t new_len);

/* Truncate to 0 and release the id. */
int had_kvpt_seq_free(had_kvpt *h, int32_t seq);

int had_kvpt_seq_len(const had_kvpt *h, int32_t seq, int32_t *len);

/* Write the page-table rows and lengths of n sequences:
 * page_table host int32[n][max_pages] (unused entries = -1),
 * seq_lens host int32[n].  HAD_ERR_INVALID_ARG if a sequence holds more
 * than max_pages pages. */
int had_kvpt_export(const had_kvpt *h, const int32_t *seqs, int32_t n,
                    int32_t *page_table, int32_t max_pages, int32_t *seq_lens);

/* The pool's page count and page size. */
int had_kvpt_info(const had_kvpt *h, int32_t *num_pages, int32_t *page_size);

/* Number of free pages and of pages with a reference. */
int had_kvpt_stats(const had_kvpt *h, int32_t *n_free, int32_t *n_used);

/* ----------------------------------------------------------------------
 * State slots of the linear-attention (GDN) layers: reference-counted ids
 * into a caller-owned float32 pool [n_slots][H][d_v][d_k].  A sequence's
 * current state is addressed by index (current_input_indices, zubnet.ai ¶2):
 * a cached checkpoint is shared by retaining its id and is never written;
 * a step reads slot in_idx and writes a fresh slot out_idx (copy-on-write
 * by index, no tensor copy).  Same free-list policy as the pages.
 * ---------------------------------------------------------------------- */
typedef struct had_slots had_slots;

int had_slots_create(int32_t n_slots, const int32_t *free_order, had_slots **out);
int had_slots_destroy(had_slots *h);
int had_slots_acquire(had_slots *h, int32_t *slot);   /* refcount = 1 */
int had_slots_retain(had_slots *h, int32_t slot);     /* HAD_ERR_BAD_SLOT if not held */
int had_slots_release(had_slots *h, int32_t slot);    /* back to the free list at 0 */
int had_slots_stats(const had_slots *h, int32_t *n_free, int32_t *n_used);

/* Accept the first `accepted` of T verified draft tokens of seq (its length
 * includes the T drafts).  KV: truncate to length - T + accepted.  State:
 * *current_slot = in_slot if accepted == 0 else out_slots[accepted - 1];
 * every other out slot is released in draft order, then in_slot is released
 * if accepted > 0 and in_slot >= 0 (in_slot = -1 is the zero state).  All
 * preconditions (distinct held out slots, in_slot held, 0 <= accepted <= T,
 * length >= T) are checked first; on error nothing changes.  Rollback is an
 * index update only: no device memory is touched (24-ai.news, "Mamba State
 * Update": O(1) pointer update).  out_slots: host int32[T]. */
int had_spec_rollback(had_kvpt *kv, had_slots *slots, int32_t seq, int32_t T,
                      int32_t accepted, int32_t in_slot, const int32_t *out_slots,
                      int32_t *current_slot);

/* ----------------------------------------------------------------------
 * Hybrid prefix cache: a radix tree over token ids whose nodes hold the KV
 * pages of their token span and, where a state was saved, a GDN state slot
 * (the checkpoint of the recurrent layers at exactly that prefix length):
 * the host-side half of hybrid prefix caching (24-ai.news TokenSpeed
 * article, optimisation list; zubnet.ai ¶2, reuse of cached checkpoints
 * without writing them).  A hybrid model can resume only where both the KV
 * and the recurrent state exist, so a match ends at the deepest node on the
 * query's path that carries a slot.
 *
 * The cache holds its own references on pages (had_kvpt_page_retain) and
 * slots (had_slots_retain); callers keep and release theirs as usual.
 * Matched pages and slots are shared, never written by the cache's users:
 * a request appends through had_kvpt_reserve (copy-on-write of a shared
 * partial page) and writes its states to fresh slots.
 * ---------------------------------------------------------------------- */
typedef struct had_radix had_radix;

/* The cache works on kv and slots, which must outlive it. */
int had_radix_create(had_kvpt *kv, had_slots *slots, had_radix **out);
/* Releases every page and slot reference the cache holds. */
int had_radix_destroy(had_radix *r);

/* Longest prefix of tokens[0..n) that is cached and ends at a checkpoint.
 * *matched: its length (0 when none); *slot: its state slot (-1 for length
 * 0: the zero state); pages: host int32[max_pages] receives the
 * ceil(*matched / page_size) page ids holding the prefix's KV (valid rows:
 * the first *matched positions; the caller may create a sequence on them
 * with had_kvpt_seq_create_from).  *lock receives a handle that keeps the
 * matched path from eviction until had_radix_unlock (-1 when *matched is 0).
 * HAD_ERR_CAPACITY if max_pages is too small (nothing changes). */
int had_radix_match(had_radix *r, const int32_t *tokens, int32_t n, int32_t *matched, int32_t *slot,
                    int32_t *pages, int32_t max_pages, int32_t *lock);
int had_radix_unlock(had_radix *r, int32_t lock);

/* Cache tokens[0..n) with their pages (host int32[ceil(n / page_size)],
 * every page held; the positions already cached keep the cache's pages) and
 * slot (the state after token n-1; -1 for none).  The cache takes its own
 * references on what it keeps.  *new_tokens (optional): tokens not cached
 * before. */
int had_radix_insert(had_radix *r, const int32_t *tokens, int32_t n, const int32_t *pages, int32_t slot,
                     int32_t *new_tokens);

/* Evict least-recently-used unlocked entries until the page pool has at
 * least min_free_pages free pages and the slot pool min_free_slots free
 * slots, or nothing evictable is left: leaves go first (their pages and
 * slot), then checkpoints of inner nodes (their slot only).
 * *n_evicted (optional): entries evicted. */
int had_radix_evict(had_radix *r, int32_t min_free_pages, int32_t min_free_slots, int32_t *n_evicted);

/* Nodes (root excluded), cached tokens, checkpoints, and the match
 * counters: queried tokens and matched tokens over all had_radix_match
 * calls (the cache hit rate is their ratio). */
int had_radix_stats(const had_radix *r, int32_t *n_nodes, int64_t *cached_tokens, int32_t *n_checkpoints,
                    int64_t *queried_tokens, int64_t *matched_tokens);

/* ======================================================================
 * kv_page_table -- device helpers
 * ====================================================================== */
typedef struct {
  int32_t num_pages;  /* pages in each pool                    */
  int32_t H_kv;       /* KV heads                              */
  int32_t page_size;  /* tokens per page (P)                   */
  int32_t head_dim;   /* D                                     */
} had_kv_layout;
/* Pools: K and V, bf16 [num_pages][H_kv][page_size][head_dim] each, one
 * pair per attention layer.  One (page, head) is a contiguous block of
 * page_size * head_dim * 2 bytes. */

/* Copy whole pages d_src[i] -> d_dst[i] (all heads) in both pools, i < n
 * (n <= 65535).  This is the device half of copy-on-write: the (src, dst) of
 * the triple from had_kvpt_reserve (zubnet.ai TokenSpeed article, second
 * paragraph: cached pages reused without being written).
 * d_src, d_dst: DEVICE int32 [n], read when the copy runs, so a captured
 * graph can be replayed with new pairs.  A pair with d_src[i] == -1 is an
 * unused entry and copies nothing (a graph can carry a fixed number of
 * entries).  Checked on the device, pair by pair, before any byte moves: a
 * pair with an id outside [0, num_pages) sets HAD_DERR_PAGE, a pair whose
 * destination is the source of an active pair (itself included) or the
 * destination of an earlier active pair sets HAD_DERR_COPY; such a pair is
 * skipped, the others are copied.  d_err: optional device word.
 * had_kv_check_copy_pages runs the same checks on host copies of the arrays
 * (the binding calls it when the environment sets HAD_DEBUG=1). */
int had_kv_copy_pages(const had_kv_layout *L, void *k_pool, void *v_pool,
                      const int32_t *d_src, const int32_t *d_dst, int32_t n, int32_t *d_err,
                      void *stream);

/* The checks of had_kv_copy_pages on host arrays src, dst (int32 [n]):
 * HAD_ERR_INVALID_ARG names the first pair that the device would skip. */
int had_kv_check_copy_pages(int32_t num_pages, const int32_t *src, const int32_t *dst, int32_t n);

/* Raw append: write t_new tokens per sequence at positions
 * seq_lens[s] - t_new + j (seq_lens already include them).
 * k_new, v_new: device bf16 [n_seqs][t_new][H_kv][head_dim];
 * d_page_table: device int32 [n_seqs][max_pages]; d_seq_lens: device int32. */
int had_kv_append(const had_kv_layout *L, void *k_pool, void *v_pool,
                  const int32_t *d_page_table, int32_t max_pages,
                  const int32_t *d_seq_lens, const void *k_new, const void *v_new,
                  int32_t n_seqs, int32_t t_new, int32_t *d_err, void *stream);

/* ======================================================================
 * qk_norm_rope_gate -- fused prologue of a full-attention layer
 * (zubnet.ai ¶2: QK-RMSNorm + partial RoPE + gate split fused into one
 * kernel with intermediates in registers).
 *
 * For each sequence s, new token j (position pos = seq_lens[s] - T + j) and
 * head:
 *   q    = RMSNorm(qg[s][j][hq][0][:]) * w_q,  gate = qg[s][j][hq][1][:]
 *   k    = RMSNorm(k[s][j][h][:]) * w_k,       v passed through
 *   RMSNorm(x) = x / sqrt(mean(x^2) + eps)     (fp32)
 *   then the first rotary_dim dims of q and k are rotated, pairs
 *   (i, i + rotary_dim/2), angle pos * rope_base^(-2i/rotary_dim) (fp64)
 *   (RoFormer rotary embedding applied to a prefix of the head).
 * Writes q_out, gate_out (bf16, round to nearest even) and k, v into the
 * KV pools at the page slot of pos.
 * ====================================================================== */
typedef struct {
  int32_t n_seqs, T, H_q, H_kv, head_dim, rotary_dim; /* head_dim in {64,128,256}, rotary_dim even, <= head_dim */
  double rope_base;                                   /* e.g. 10000                                            */
  float eps;                                          /* e.g. 1e-6                                             */
  int32_t num_pages, page_size, max_pages;            /* pool pages, tokens per page, page_table row stride    */
} had_qknrg_desc;

typedef struct {
  const void *qg;            /* bf16 [n_seqs][T][H_q][2][head_dim]  (q then gate)  */
  const void *k;             /* bf16 [n_seqs][T][H_kv][head_dim]                   */
  const void *v;             /* bf16 [n_seqs][T][H_kv][head_dim]                   */
  const float *w_q, *w_k;    /* fp32 [head_dim]                                    */
  const int32_t *page_table; /* int32 [n_seqs][max_pages]                          */
  const int32_t *seq_lens;   /* int32 [n_seqs], lengths including the T new tokens */
  void *k_pool, *v_pool;     /* bf16 pools (layout above), written                 */
  void *q_out, *gate_out;    /* bf16 [n_seqs][T][H_q][head_dim], written           */
  int32_t *d_err;            /* optional device flag word                          */
} had_qknrg_ptrs;

int had_qk_norm_rope_gate(const had_qknrg_desc *d, const had_qknrg_ptrs *p, void *stream);

/* ======================================================================
 * decode_attn -- split-K GQA decode attention over the paged KV cache
 *
 * For sequence s, query token j < q_len and query head hq (KV head
 * h = hq / (H_q / H_kv)):  n = seq_lens[s] - q_len + j + 1 keys are visible
 * (causal inside the draft), and
 *   out[s][j][hq] = softmax_t(sm_scale * q . K[t]) @ V[t],  t < n,
 * with K/V read through the page table.  Full-attention layers of the hybrid
 * model (24-ai.news, model paragraph) at contexts up to 1M tokens
 * (long-context table).
 *
 * Work is split over the context ("split-K"): of the n pages that
 * max_seq_len can reach (N = n * page_size / 8 tiles of 8 tokens), work
 * unit (s, h, split i of ns) covers, below 16 rows, the tiles
 * [i*b + min(i, r), (i+1)*b + min(i+1, r)) with b = N / ns, r = N % ns
 * (balanced to within one tile) and, at 16 rows or more, the pages
 * [i*n/ns, (i+1)*n/ns) (within one page); pages_per_split of
 * the plan = ceil(n/ns), at most 512, and below 16 rows at most 511 when
 * ns > 1 (a tile range can touch one page more, and one split reads at most
 * 512); every seq_lens[s] must lie within the n pages (n * page_size tokens),
 * else HAD_DERR_SEQLEN is set and the sequence is skipped (nothing written for
 * it, the fused prologue's K/V rows included).  A unit writes an unnormalised partial
 * (o, m, l) to the workspace; a second kernel merges the partials by
 * log-sum-exp and writes bf16 (round to nearest even).  Query rows per KV
 * head = q_len * (H_q / H_kv); below 16 rows a VALU kernel runs, at 16 or
 * more a bf16 MFMA kernel.
 *
 * Workspace (caller-allocated device memory, >= had_decode_attn_workspace_bytes):
 *   ws_o  fp32 [n_seqs][H_kv][num_splits][rows][head_dim]
 *   ws_ml fp32 [n_seqs][H_kv][num_splits][rows][2]   (m, l)
 *   ws_q  bf16 [n_seqs][q_len][H_q][head_dim]         (had_decode_attn_layer only)
 * starting at the workspace base, ws_ml right after ws_o, ws_q at the next
 * 256-byte boundary.  Row r = j * G + g
 * is query j, head h * G + g.  m is in base-2 units: m = max over the split
 * of sm_scale * log2(e) * q.k; l = sum of 2^(that - m); o = sum of
 * 2^(that - m) * v.  An empty split has m = -inf, l = 0, o = 0.
 * ====================================================================== */
typedef struct {
  int32_t n_seqs, q_len, H_q, H_kv, head_dim; /* head_dim in {64,128,256}; H_q % H_kv == 0           */
  int32_t num_pages, page_size, max_pages;    /* pool pages; page_size a multiple of 8 in [8, 256]     */
  float sm_scale;                             /* usually 1/sqrt(head_dim)                            */
  int32_t max_seq_len;                        /* host bound on every seq_lens[s]; 0 = max_pages*page_size */
  int32_t num_splits;                         /* 0 = choose automatically                            */
  int32_t flags;                              /* HAD_ATTN_* bits                                     */
} had_attn_desc;

/* Work inside a split is handed to the waves dynamically by default, which
 * balances waves that share a SIMD but makes the fp32 summation order (and
 * so the last bits of the output) depend on timing.  With this flag every
 * wave takes a fixed stride of tiles: the output bits are a function of the
 * inputs and the split plan only. */
#define HAD_ATTN_DETERMINISTIC 1

/* The merge multiplies the attention output by sigmoid(gate) elementwise
 * (fp32, before the bf16 rounding of out) -- the gated attention output of
 * the hybrid model's full-attention layers.  had_decode_attn and
 * had_decode_attn_cascade read the gate from had_attn_ptrs.gate (NULL is an
 * error); had_decode_attn_layer takes the second half of qg; the split entry
 * points (_partial, _combine, _layer_partial) reject the flag. */
#define HAD_ATTN_GATED_OUTPUT 4

typedef struct {
  const void *q;             /* bf16 [n_seqs][q_len][H_q][head_dim]         */
  const void *k_pool, *v_pool;
  const int32_t *page_table; /* int32 [n_seqs][max_pages]                   */
  const int32_t *seq_lens;   /* int32 [n_seqs] (include the q_len tokens)   */
  void *workspace;
  size_t workspace_bytes;
  void *out;                 /* bf16 [n_seqs][q_len][H_q][head_dim]         */
  int32_t *d_err;            /* optional                                    */
  const void *gate;          /* bf16 [n_seqs][q_len][H_q][head_dim], read   *
                              * with HAD_ATTN_GATED_OUTPUT only (the gate   *
                              * that had_qk_norm_rope_gate splits off)      */
} had_attn_ptrs;

/* Split plan for desc: number of splits and ceil(pages / splits) (both
 * depend on the descriptor only, never on device data). */
int had_decode_attn_plan(const had_attn_desc *d, int32_t *num_splits, int32_t *pages_per_split);
size_t had_decode_attn_workspace_bytes(const had_attn_desc *d);
int had_decode_attn(const had_attn_desc *d, const had_attn_ptrs *p, void *stream);

/* The two halves of had_decode_attn, for callers that move or inspect the
 * partials between them (e.g. a context-parallel split of one sequence over
 * several devices exchanges the (o, m, l) partials before merging).
 * had_decode_attn_partial writes the workspace only (p->out is ignored);
 * had_decode_attn_combine reads num_splits partials in the workspace layout
 * above and writes out. */
int had_decode_attn_partial(const had_attn_desc *d, const had_attn_ptrs *p, void *stream);
int had_decode_attn_combine(const had_attn_desc *d, int32_t num_splits,
                            const void *workspace, void *out, void *stream);

/* ======================================================================
 * decode_attn_cascade -- decode attention for a batch sharing a prefix
 *
 * The sequences of a batch that forked one cached prefix (page aliasing:
 * zubnet.ai ¶2 and 24-ai.news, hybrid prefix caching) share its pages; here
 * those pages are streamed once for the query rows of every sequence (MFMA
 * kernel: rows = n_seqs x q_len x H_q/H_kv per KV head) instead of once per
 * sequence, each sequence's own pages after the prefix are streamed by the
 * usual split-K kernel, and the ordinary merge combines both sets of
 * partials.  Output: as had_decode_attn (same operation; the sums differ in
 * order only).
 *
 * px->prefix_pages whole pages (>= 1) form the shared prefix; px's page list
 * must equal the first prefix_pages entries of every sequence's page-table
 * row (not checked on the device: had_attn_check_prefix checks host copies,
 * and the binding runs it when HAD_DEBUG=1), and every sequence must see the whole prefix:
 * seq_lens[s] - q_len >= prefix_pages * page_size (HAD_DERR_SEQLEN in d_err
 * otherwise).  A prefix page still being written (a shared partial page) is
 * not part of it: such a page belongs to each sequence after copy-on-write.
 * Workspace: >= had_decode_attn_cascade_workspace_bytes(d, px) bytes, layout
 * of had_decode_attn's ws_o / ws_ml with the prefix splits first (returns 0
 * for an invalid descriptor).
 *
 * Suffix pass below 16 rows (n_seqs <= 64, suffix plan <= 510 pages,
 * num_splits = 0): the suffixes differ in length, so instead of the same
 * number of splits per sequence the pass runs G work units per KV head
 * (G = max(n_seqs, 256 / H_kv)); every sequence with a suffix tile gets one
 * unit and the rest go to the sequences in proportion to their suffix length
 * (8-token tiles from token prefix_pages * page_size on, the floor of the
 * proportional share), each unit taking an equal range of its sequence's
 * tiles.  The units are read from seq_lens on the device, so the shares
 * follow the lengths of every step (and a captured graph).  Each
 * sequence's row of the workspace has slots for G suffix partials, of which
 * its own share is written; had_decode_attn_cascade_combine merges exactly
 * those.
 * ====================================================================== */
typedef struct {
  int32_t prefix_pages;              /* whole pages shared by every sequence (>= 1)  */
  const int32_t *prefix_page_table;  /* device int32 [prefix_pages]: their ids, in order */
} had_attn_prefix;

size_t had_decode_attn_cascade_workspace_bytes(const had_attn_desc *d, const had_attn_prefix *px);

/* Host check of the cascade's page-list precondition on host copies:
 * page_table int32 [n_seqs][max_pages], prefix int32 [prefix_pages].
 * HAD_ERR_INVALID_ARG names the first sequence whose row does not begin with
 * the prefix's pages (e.g. a prefix page replaced by copy-on-write). */
int had_attn_check_prefix(int32_t n_seqs, int32_t max_pages, const int32_t *page_table, int32_t prefix_pages,
                          const int32_t *prefix);
int had_decode_attn_cascade(const had_attn_desc *d, const had_attn_prefix *px, const had_attn_ptrs *p,
                            void *stream);

/* The cascade's split plan: *prefix_splits partials of the prefix pass come
 * first in each (sequence, KV head) slot of the workspace, then
 * *suffix_splits slots of the suffix pass (G when the suffix units are
 * shared out by length, see above). */
int had_decode_attn_cascade_plan(const had_attn_desc *d, const had_attn_prefix *px, int32_t *prefix_splits,
                                 int32_t *suffix_splits);

/* The cascade's passes without the merge: passes = 1 (prefix pass), 2
 * (suffix pass) or 3 (both) write their partials into the workspace (layout
 * above; p->out and p->gate are ignored, HAD_ATTN_GATED_OUTPUT is rejected);
 * had_decode_attn_cascade_combine with the same arguments finishes (not
 * had_decode_attn_combine: with the suffix shared out by length not every
 * slot is written).  For callers that schedule or time the passes
 * separately. */
int had_decode_attn_cascade_partial(const had_attn_desc *d, const had_attn_prefix *px, const had_attn_ptrs *p,
                                    int32_t passes, void *stream);
/* The cascade's merge alone: out (and the gate, with HAD_ATTN_GATED_OUTPUT)
 * from the partials both passes wrote; ptrs as had_decode_attn_cascade. */
int had_decode_attn_cascade_combine(const had_attn_desc *d, const had_attn_prefix *px, const had_attn_ptrs *p,
                                    void *stream);

/* ======================================================================
 * decode_attn_layer -- qk_norm_rope_gate and decode_attn in one pass
 *
 * Below 16 query rows per KV head the prologue of a full-attention layer
 * runs inside the split-K partial kernel (the pages fuse the prologue's five
 * steps into one kernel: zubnet.ai ¶2; here it is fused one step further,
 * into the attention): every work unit normalises and rotates its own query
 * rows, the unit whose split holds the last position normalises and rotates
 * the T new keys, writes the new K/V rows to the pools and adds the new
 * tokens to its partial from on-chip copies; then the usual merge writes
 * out.  The same holds at 16..128 rows on the MFMA path when pages hold a
 * multiple of 32 tokens (16..64 rows only at head_dim >= 128), the rotary
 * dims are 0, 64 or a multiple of 128, and qg, w_q, w_k, gate_out and q_out
 * are 16-byte aligned: every unit forms its query rows in the MFMA operand
 * registers.  Other MFMA shapes run the prologue once as
 * had_qk_norm_rope_gate, writing q to pp->q_out or, when that is NULL, to
 * the workspace's ws_q block.
 *
 * Results: out as had_decode_attn with q = the q_out of had_qk_norm_rope_gate
 * (the attention sums differ in order only); gate_out, the pools and (when
 * non-NULL) q_out as had_qk_norm_rope_gate -- the same bits, except that
 * where the MFMA path forms q inline the RMSNorm's fp32 sum of squares runs
 * in another order, so an element of q may differ by one bf16 ulp.
 *
 * d and pd describe the same layer (n_seqs, T = q_len, heads, head_dim, pool
 * geometry must agree, else HAD_ERR_INVALID_ARG); pp supplies every pointer
 * (pp->q_out may be NULL; pp->d_err is used for both halves); workspace as
 * had_decode_attn (had_decode_attn_workspace_bytes(d)).  T <= 8
 * (HAD_ERR_UNSUPPORTED_SHAPE otherwise).
 * ====================================================================== */
int had_decode_attn_layer(const had_attn_desc *d, const had_qknrg_desc *pd, const had_qknrg_ptrs *pp,
                          void *workspace, size_t workspace_bytes, void *out, void *stream);

/* Allocation-free form of had_decode_attn_layer, for callers that cannot
 * allocate device memory: code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc.  The split-K workspace is an array of
 * HAD_STATIC_WORKSPACE_BYTES inside the library, one per GPU, held from the
 * time the library's kernels are loaded on that GPU until the process ends;
 * the caller passes only inputs and outputs.  Same operation, arguments and
 * results as had_decode_attn_layer.  The call allocates nothing; the first
 * call on each device looks up that device's array address
 * (hipGetSymbolAddress), so make it outside graph capture.
 * HAD_ERR_WORKSPACE_TOO_SMALL when had_decode_attn_workspace_bytes(d) exceeds
 * the array (e.g. 64 query rows x 256 splits x head_dim 256 need 17 MB).
 * Every call on one GPU uses that GPU's single array and leaves its partials
 * there: calls that overlap in time on one GPU (two streams, two host
 * threads) race on it and must be ordered by the caller. */
#define HAD_STATIC_WORKSPACE_BYTES (32u << 20)
int had_decode_attn_layer_static(const had_attn_desc *d, const had_qknrg_desc *pd, const had_qknrg_ptrs *pp,
                                 void *out, void *stream);

/* Its first half: the prologue and the partials only (workspace layout of
 * had_decode_attn); had_decode_attn_combine finishes. */
int had_decode_attn_layer_partial(const had_attn_desc *d, const had_qknrg_desc *pd, const had_qknrg_ptrs *pp,
                                  void *workspace, size_t workspace_bytes, void *stream);

/* ======================================================================
 * gdn_state_update -- gated delta rule on slot-addressed states
 *
 * For sequence s and head h, with S (d_v x d_k) read from
 * state_pool[in_idx[s]][h] (zero when in_idx[s] == -1), for t < T:
 *   S <- alpha_t * S (I - beta_t k_t k_t^T) + beta_t v_t k_t^T
 *   o[s][t][h] = q_scale * S q_t,  S written to state_pool[out_idx[s][t]][h]
 * (Gated DeltaNet layers of the hybrid model, 24-ai.news model paragraph;
 * recurrence as in Yang, Kautz & Hatamizadeh, ICLR 2025; states addressed by
 * index, zubnet.ai ¶2 and 24-ai.news "Mamba State Update").  fp32 state and
 * arithmetic.  With T > 1 every token's state is a checkpoint (speculative
 * verify); the caller picks the kept one by index (had_spec_rollback).
 * Preconditions (not checked on device): no slot is written by two
 * (s, t) pairs, and no slot written by the call is read by another sequence
 * of the same call.  in_idx[s] == out_idx[s][0] is allowed only when T == 1.
 * ====================================================================== */
typedef struct {
  int32_t n_seqs, T, H, d_k, d_v; /* d_k, d_v in {64, 128}; 1 <= T <= 8 */
  int32_t n_slots;
  float q_scale;                  /* 1 for the plain recurrence          */
  int32_t flags;                  /* HAD_GDN_* bits                      */
} had_gdn_desc;

/* alpha[] and beta[] hold the raw gate values g and b of each (token, head):
 * the kernel forms alpha = exp(g) (g <= 0, the log decay) and
 * beta = 1 / (1 + exp(-b)) in fp32 (the Gated DeltaNet parameterisation). */
#define HAD_GDN_RAW_GATES 1

typedef struct {
  float *state_pool;         /* fp32 [n_slots][H][d_v][d_k]              */
  const int32_t *in_idx;     /* int32 [n_seqs]  (-1 = zero state)         */
  const int32_t *out_idx;    /* int32 [n_seqs][T]                         */
  const void *q, *k;         /* bf16 [n_seqs][T][H][d_k]                  */
  const void *v;             /* bf16 [n_seqs][T][H][d_v]                  */
  const float *alpha, *beta; /* fp32 [n_seqs][T][H]                       */
  float *o;                  /* fp32 [n_seqs][T][H][d_v], written         */
  int32_t *d_err;            /* optional                                  */
} had_gdn_ptrs;

int had_gdn_state_update(const had_gdn_desc *d, const had_gdn_ptrs *p, void *stream);

/* Host check of the slot preconditions that the GDN kernels do not check
 * on the device (two sequences racing on one slot is not visible there), on
 * host copies of the index arrays: every id in range (in_idx >= -1), no
 * slot written twice, no slot written by one sequence and read by another,
 * and in_idx[s] equal to one of its own out slots only when allow_in_place
 * (had_gdn_state_update with T == 1, had_gdn_prefill).  out_idx: host
 * int32[n_seqs][T] (T = 1 for the prefill).  HAD_ERR_BAD_SLOT names the
 * first violation.  A debugging aid: the binding runs it before every GDN
 * call when the environment sets HAD_DEBUG=1. */
int had_gdn_check_slots(int32_t n_seqs, int32_t T, int32_t n_slots, const int32_t *in_idx, const int32_t *out_idx,
                        int32_t allow_in_place);

/* ======================================================================
 * gdn_prefill -- the same recurrence over whole prompts, chunk-parallel
 *
 * Sequence s owns tokens cu_seqlens[s] .. cu_seqlens[s+1]-1 of the packed
 * inputs; it starts from slot in_idx[s] (zero state for -1), runs the gated
 * delta rule over all of its tokens (as had_gdn_state_update would, token
 * by token), writes o for every token and its final state, fp32, to slot
 * out_idx[s] only.  A sequence with no token copies its input state;
 * in_idx[s] == out_idx[s] (in place) is allowed.  This is the GDN half of a
 * prefill: the turn inputs and the long first turn of the agentic loop
 * (24-ai.news TokenSpeed article, agentic workload; GDN layers and their
 * state checkpoints: same article, model paragraph, and zubnet.ai ¶2).
 *
 * Evaluation: chunks of 64 tokens in the WY / UT form of the delta rule
 * (Yang et al., NeurIPS 2024, "Parallelizing Linear Transformers with the
 * Delta Rule over Sequence Length"; gated form in the Gated DeltaNet paper):
 * a chunk-parallel kernel forms each chunk's triangular solve and
 * state-independent products, then a scan kernel carries the state across
 * the chunks of a sequence (MFMA; state kept in fp32, its matrix products
 * in split bf16 pairs).  For long prompts the scan runs in segments side by
 * side: each segment's map S -> S PI + SE (PI the d_k x d_k product of the
 * chunks' transitions, SE the state reached from zero) is scanned first,
 * the segments' start states are chained (fp32), and the segments are
 * scanned again from their start states.  The result equals the
 * token-by-token recurrence up to rounding (fp32 accumulation; relative
 * error ~1e-5 per chunk).
 *
 * Shapes: d_k, d_v in {64, 128}; any H; 0 <= length <= max_len.
 * state_pool, q, k, v and the workspace must be 16-byte aligned
 * (HAD_ERR_INVALID_ARG otherwise).
 * Preconditions (not checked on device): no slot is written by two
 * sequences, and no slot a sequence writes is read by another sequence.
 * Device errors: HAD_DERR_SLOT (slot out of range: the sequence is skipped),
 * HAD_DERR_SEQLEN (cu_seqlens not non-decreasing, or a length above
 * max_len: skipped).
 * ====================================================================== */
typedef struct {
  int32_t n_seqs, H, d_k, d_v;
  int32_t n_slots;
  int32_t max_len;           /* host bound on every sequence's length      */
  float q_scale;
  int32_t flags;             /* HAD_GDN_RAW_GATES                          */
  int32_t n_segments;        /* scan segments (>= 0; capped at the chunk    *
                              * count).  0 = automatic: g = min(chunks/32, *
                              * 512 / (n_seqs x H x d_v/16)), one segment  *
                              * when g < 3                                 */
} had_gdn_prefill_desc;

typedef struct {
  float *state_pool;         /* fp32 [n_slots][H][d_v][d_k]                */
  const int32_t *in_idx;     /* int32 [n_seqs] (-1 = zero state)           */
  const int32_t *out_idx;    /* int32 [n_seqs]                             */
  const int32_t *cu_seqlens; /* int32 [n_seqs + 1], device, token offsets  */
  const void *q, *k;         /* bf16 [N][H][d_k], N = cu_seqlens[n_seqs]    */
  const void *v;             /* bf16 [N][H][d_v]                           */
  const float *alpha, *beta; /* fp32 [N][H] (raw g, b with RAW_GATES)      */
  float *o;                  /* fp32 [N][H][d_v], written                  */
  void *workspace;           /* had_gdn_prefill_workspace_bytes(d) bytes   */
  size_t workspace_bytes;
  int32_t *d_err;            /* optional                                   */
} had_gdn_prefill_ptrs;

/* Workspace: per (sequence, chunk of 64 tokens up to max_len, head) the
 * chunk's solve results, and with segments per (sequence, segment, head)
 * three fp32 d_k-wide blocks (PI, SE, the start state); 0 for an invalid
 * descriptor. */
size_t had_gdn_prefill_workspace_bytes(const had_gdn_prefill_desc *d);
int had_gdn_prefill(const had_gdn_prefill_desc *d, const had_gdn_prefill_ptrs *p, void *stream);

#ifdef __cplusplus
}
#endif
#endif /* HAD_H */
