/*
 * rc.h — C ABI of the prefix-shared KV attention library (gfx950 / MI355X).
 *
 * The operations follow two pages:
 *   [PC]  "Prompt Caching" glossary (Ultralytics): the problem statement.
 *         Section "How prompt caching works": prefill computes one key and one
 *         value per prompt token per layer; every decoded token attends to all
 *         of them; because attention is causal the K/V of an identical prefix
 *         are identical, so a cached copy replaces the recompute and only the
 *         new tokens run.  Opening paragraph: reuse needs an exactly identical
 *         prefix.  Closing list: a hit leaves next-token scores unchanged up to
 *         floating-point rounding.
 *   [SG]  "SGLang: Efficient Execution of Structured Language Model Programs"
 *         summary (unite.ai): section "SGLang: programming model", RadixAttention
 *         bullet (KV kept in a radix tree used for match / insert / evict, LRU
 *         policy), the `fork` primitive, and the nine-step radix tree example
 *         (new turns inserted as nodes; nodes split so sessions share a prompt).
 *
 * Conventions for every call
 *   - Tensors are dense, row-major, caller-owned.  "device" pointers are HIP
 *     device memory, "host" pointers are ordinary host memory.  The library
 *     never allocates or frees device memory; it borrows pointers for the call.
 *   - GPU calls only enqueue work on `stream` (a hipStream_t passed as void*,
 *     NULL = the null stream) and return; the caller keeps buffers alive until
 *     that work completes.
 *   - Arguments are validated on the host before anything is launched; a
 *     failing call returns a non-zero rc_status, launches nothing, changes
 *     nothing, and rc_last_error() describes the failure (thread-local).
 *   - Indices read from device memory (slots, table entries, plan entries) are
 *     bounds-checked inside the kernels: an invalid one is never dereferenced;
 *     the affected key is treated as absent and a bit is OR-ed into the device
 *     error word if one was registered with rc_set_error_word().
 *   - Layouts: q, o            [tokens, Hq, D]
 *              k_new, v_new    [tokens, Hkv, D]
 *              k_pool, v_pool  [pool_slots, Hkv, D]   (page size: one token)
 *              req_to_token    [rows, stride] int32   (slot of position j of a
 *                                                      request's context)
 *   - Grouped-query attention: query head h reads kv head h / (Hq / Hkv).
 *   - sm_scale (the softmax scale, usually 1/sqrt(head_dim)) must be finite
 *     and positive, else RC_ERR_ARG.
 *   - Causal alignment is by absolute position: new token i of a request with
 *     a cached prefix of P tokens is at position P+i and sees keys 0..P+i.
 */
#ifndef RC_H
#define RC_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum rc_status {
  RC_OK = 0,
  RC_ERR_ARG = 1,      /* null pointer, negative size, malformed argument        */
  RC_ERR_SHAPE = 2,    /* head counts / head_dim not supported or inconsistent  */
  RC_ERR_DTYPE = 3,    /* unsupported dtype                                     */
  RC_ERR_RANGE = 4,    /* an index or length outside its documented range       */
  RC_ERR_NOMEM = 5,    /* the KV pool has too few free slots (host tree calls)  */
  RC_ERR_HIP = 6,      /* a HIP runtime call or kernel launch failed            */
  RC_ERR_INTERNAL = 7
} rc_status;

typedef enum rc_dtype { RC_F32 = 0, RC_BF16 = 1 } rc_dtype;

/* Model-side shape shared by the KV pool and the attention calls.
 * num_q_heads % num_kv_heads == 0, group = num_q_heads / num_kv_heads <= 128,
 * head_dim in {64, 128}. */
typedef struct rc_shape {
  int32_t dtype;        /* rc_dtype of q, k, v, pools and o                     */
  int32_t num_q_heads;
  int32_t num_kv_heads;
  int32_t head_dim;
  int64_t pool_slots;   /* rows of k_pool / v_pool                              */
  int32_t page_size;    /* 0 or 1: req_to_token holds one slot per position.   */
                        /* A power of two up to 1024: the pool is made of pages */
                        /* of page_size consecutive slots (pool_slots a        */
                        /* multiple of it) and req_to_token holds one page id  */
                        /* per page_size positions (its stride counts pages): */
                        /* position p reads slot page(p / page_size) *         */
                        /* page_size + p % page_size ("Prompt Caching"        */
                        /* glossary, serving engines: paged KV blocks).        */
                        /* Slot arguments (new_slots, rc_kv_store) stay per   */
                        /* token.                                              */
  int32_t reserved;     /* 0                                                    */
} rc_shape;

/* Bits OR-ed into the device error word. */
#define RC_DEVERR_SLOT 1    /* a slot outside [0, pool_slots)                    */
#define RC_DEVERR_TABLE 2   /* a table position outside [0, stride)              */
#define RC_DEVERR_LENGTH 4  /* extend_len > max_extend or a negative length      */
#define RC_DEVERR_PLAN 8    /* a malformed plan entry                            */
#define RC_DEVERR_LABEL 16  /* a label id outside [0, vocab) or an option count  */
                            /* outside [1, n_labels]                             */

const char* rc_last_error(void);
const char* rc_version(void);

/* Register a device int32 that kernels OR RC_DEVERR_* bits into (NULL = off).
 * Process-wide; not thread-safe against concurrent GPU calls. */
rc_status rc_set_error_word(int32_t* device_word);

/* Copy a rectangle of a host req_to_token table to its device copy on       */
/* `stream`: rows [row0, row0 + n_rows), entries [col0, col1) of each.  Both */
/* tables are row-major int32 with host_stride / dev_stride entries a row.   */
/* One asynchronous 2D copy: the host table should be pinned (else the copy */
/* is staged and synchronous) and must not change until the stream has run */
/* it.  Lets a caller upload only the entries rc_radix_emit_rows changed     */
/* (its first_changed output) instead of whole rows.  Bad sizes or an empty  */
/* rectangle's negative extents fail with RC_ERR_ARG; copy errors with       */
/* RC_ERR_HIP.                                                                */
rc_status rc_upload_table_rows(int32_t* dev_table, int64_t dev_stride, const int32_t* host_table,
                               int64_t host_stride, int64_t row0, int64_t n_rows, int64_t col0, int64_t col1,
                               void* stream);

/* ------------------------------------------------------------------------ */
/* KV-pool scatter  [PC] "How prompt caching works": K and V of every token   */
/* are stored and kept for later use.                                         */
/*   k_pool[slots[i], h, :] = k_new[i, h, :] and the same for V, i < n.       */
/* A bit copy (no conversion).  Slots must be distinct within one call (else */
/* which row lands is unspecified); out-of-range slots are skipped and       */
/* flagged.  Every other pool row is left unchanged.                          */
/*   k_pool, v_pool : device, [pool_slots, Hkv, D] of shape->dtype            */
/*   k_new, v_new   : device, [n, Hkv, D]                                     */
/*   slots          : device int32 [n]                                        */
/* ------------------------------------------------------------------------ */
rc_status rc_kv_store(const rc_shape* shape, void* k_pool, void* v_pool, const void* k_new,
                      const void* v_new, const int32_t* slots, int64_t n, void* stream);

/* ------------------------------------------------------------------------ */
/* Extend attention  [PC] worked example: only the new tokens of a request    */
/* run, over the cached prefix, and give the scores of a full recompute.     */
/* For request b (table row rows[b], or b when rows is NULL), new token i <  */
/* E_b = extend_lens[b] at absolute position p = P_b + i, P_b = prefix_lens[b]*/
/*   o[s_b+i, h] = sum_{j<=p} softmax_j(sm_scale * q[s_b+i,h] . k_j) v_j,     */
/* s_b = extend_start[b]; keys j < P_b are read from the pool at slot         */
/* req_to_token[row, j]; keys P_b <= j <= p from k_new/v_new[s_b + j - P_b].   */
/*   o               : device [total_extend, Hq, D], shape->dtype             */
/*   q               : device [total_extend, Hq, D]                            */
/*   k_new, v_new    : device [total_extend, Hkv, D]                           */
/*   req_to_token    : device int32 [table_rows, stride]; only entries j < P_b */
/*                     are read                                               */
/*   rows            : device int32 [batch] or NULL; rows[b] < table_rows      */
/*   prefix_lens, extend_lens, extend_start : device int32 [batch]             */
/*   max_extend      : host bound on extend_lens (sets the grid)               */
/* Requests with E_b = 0 write nothing.  Outputs are rounded once, from fp32, */
/* to shape->dtype (round to nearest even for bf16).  Device-side checks:    */
/* P_b <= stride, row < table_rows, s_b + E_b <= total_extend (else the      */
/* request is skipped and RC_DEVERR_TABLE / RC_DEVERR_LENGTH raised).         */
/* ------------------------------------------------------------------------ */
rc_status rc_extend_attention(const rc_shape* shape, void* o, const void* q, const void* k_new,
                              const void* v_new, const void* k_pool, const void* v_pool,
                              const int32_t* req_to_token, int32_t table_rows, int64_t stride,
                              const int32_t* rows, const int32_t* prefix_lens, const int32_t* extend_lens,
                              const int32_t* extend_start, int32_t batch, int64_t total_extend,
                              int32_t max_extend, float sm_scale, void* stream);

/* ------------------------------------------------------------------------ */
/* Decode work plan.  A plan lists work items; each item is a range of KV     */
/* positions [pos_begin, pos_end) read through one table row (rep_row) and   */
/* the set of requests ("members") whose contexts contain exactly those      */
/* slots at those positions.  The decode kernel loads each item's K/V once   */
/* and computes it for every member and every query head of the group: a     */
/* prefix shared by many branches is read from HBM once per step.            */
/* Layout of the int32 plan buffer (copy it to the device as is):            */
/*   [0..8)      header {RC_PLAN_MAGIC, n_items, n_members, max_splits,        */
/*                        batch, group, chunk, max_cols}                      */
/*   items       n_items x 8 {rep_row, pos_begin, pos_end, split, member_off, */
/*                            member_cnt, flags, 0}                           */
/*   members     n_members batch indices                                       */
/*   n_splits    batch entries: partial results per request                    */
/* flags: RC_PLAN_ITEM_OWN marks a piece of its one member's own positions   */
/* (the part of its context no other request of the batch reads); only such  */
/* an item stores the current token (rc_decode_attention with k_new), so a   */
/* position other requests read is never written.                            */
/* Items with members*group > 16 come first, then the narrow ones.           */
/* The kernel clamps pos_end to seq_lens[first member]; the planners only    */
/* put a range in a shared item when it lies inside every member's context.  */
/* ------------------------------------------------------------------------ */
#define RC_PLAN_MAGIC 0x52435031 /* "RCP1" */
#define RC_PLAN_HEADER 8
#define RC_PLAN_ITEM 8
#define RC_PLAN_ITEM_OWN 1 /* item flag: the range holds its member's own positions */
/* Query columns (members x group) per item: a decode plan's items fill a    */
/* four-wave tile, a cascade extend plan's (rc_radix_plan_extend) an         */
/* eight-wave one (when the group alone is wider, an item has one member).   */
#define RC_DECODE_COLS 128
#define RC_EXTEND_SHARED_COLS 256

typedef struct rc_plan_info {
  int32_t n_items;
  int32_t n_members;
  int32_t max_splits;
  int32_t batch;
  int32_t group;       /* Hq / Hkv the plan was built for                       */
  int32_t chunk;       /* nominal positions per item (pieces are balanced and */
                       /* at most chunk + chunk/8 long)                        */
  int32_t max_cols;    /* max members*group per item (at most RC_DECODE_COLS   */
                       /* for decode plans, RC_EXTEND_SHARED_COLS for cascade  */
                       /* extend plans)                                        */
  int32_t shared_items;/* items with more than one member                       */
  int32_t narrow_begin;/* items from here on have members*group <= 16 (the plan */
                       /* lists wider items first)                              */
  int32_t narrow_first;/* 1: the decode launch deals out the narrow items before */
                       /* the wide ones (the longer-running class goes first)   */
  int64_t plan_ints;   /* length of the plan buffer in int32                    */
  int64_t unique_positions; /* sum over items of (pos_end - pos_begin)         */
  int64_t logical_positions;/* sum over requests of their context length       */
} rc_plan_info;

/* A plan without sharing: one chain of pieces per request over positions   */
/* [0, max_seq_lens[b]) of table row rows[b] (NULL rows: b).                 */
/* plan (host) receives plan_ints int32; if capacity is too small the call   */
/* returns RC_ERR_RANGE with info->plan_ints set to the size needed.         */
rc_status rc_plan_decode_unshared(int32_t batch, const int32_t* rows, const int32_t* max_seq_lens,
                                  int32_t group, int32_t chunk, int32_t* plan, int64_t capacity,
                                  rc_plan_info* info);

/* Per-step inputs of decode steps t = 0..n_steps-1 ("Prompt Caching"       */
/* glossary: each decoded token's K/V are stored and it attends over every   */
/* cached position): request b's step-t token sits at position              */
/* p = base_lens[b] + t of table row rows[b] (NULL rows: b), so             */
/*   slots[t * batch + b]    = the pool slot of position p (row[p], or       */
/*                             row[p / page_size] * page_size +              */
/*                             p % page_size with page_size > 1)             */
/*   seq_lens[t * batch + b] = p + 1 (it attends over positions [0, p])      */
/* the new_slots and seq_lens of rc_decode_attention for step t.  Host call; */
/* req_to_token is the host table [table_rows, stride].  row_entries         */
/* (nullable, batch entries): the entries each row holds (from               */
/* rc_radix_emit_rows); positions past them, or entries below 0, fail with  */
/* RC_ERR_RANGE before anything is written.                                  */
rc_status rc_decode_steps(const int32_t* req_to_token, int32_t table_rows, int64_t stride, int32_t page_size,
                          int32_t batch, const int32_t* rows, const int64_t* row_entries, const int32_t* base_lens,
                          int32_t n_steps, int32_t* slots, int32_t* seq_lens);

/* Workspace bytes rc_decode_attention needs for a plan: per member, head   */
/* and split, a partial output row in the shape's dtype (bf16 or fp32) and   */
/* an fp32 (max, sum) pair.                                                  */
int64_t rc_decode_workspace_bytes(const rc_shape* shape, const rc_plan_info* info);

/* ------------------------------------------------------------------------ */
/* Decode attention  [PC] "How prompt caching works": each new token attends */
/* to all cached keys and values.  One query token per request b:            */
/*   o[b, h] = sum_{j < L_b} softmax_j(sm_scale * q[b,h] . k_j) v_j,          */
/* L_b = seq_lens[b] counts the current token.  Keys come from the pool      */
/* through the plan's table rows.  The current token's K/V either are in the */
/* pool already (k_new = v_new = new_slots = NULL), or are passed in k_new / */
/* v_new [batch, Hkv, D]: then the call also stores them at pool slot        */
/* new_slots[b] (what rc_kv_store would do) and uses them as key L_b - 1.    */
/* That key is taken from k_new / v_new by the RC_PLAN_ITEM_OWN item holding */
/* position L_b - 1; a plan whose request has no such item (position L_b - 1 */
/* inside a shared range) reads the key from the pool and stores nothing.    */
/* Split-K: each item writes a partial (fp32 max and sum, and the output   */
/* row: for bf16 data normalised by its sum and rounded to bf16 once, for   */
/* fp32 data unnormalised fp32) per member and head; a merge kernel          */
/* combines each request's partials in fp32 in split order (deterministic,  */
/* no float atomics).                                                        */
/*   o, q          : device [batch, Hq, D]                                    */
/*   k_pool, v_pool: device [pool_slots, Hkv, D] (written only with k_new)    */
/*   req_to_token  : device int32 [table_rows, stride]                        */
/*   seq_lens      : device int32 [batch]                                     */
/*   plan_dev      : device copy of the plan buffer (info->plan_ints int32);  */
/*                   info: the summary the planner returned with it (a plan  */
/*                   with info->max_cols > RC_DECODE_COLS: RC_ERR_ARG)        */
/*   workspace     : device, >= rc_decode_workspace_bytes() bytes             */
/* ------------------------------------------------------------------------ */
rc_status rc_decode_attention(const rc_shape* shape, void* o, const void* q, void* k_pool, void* v_pool,
                              const void* k_new, const void* v_new, const int32_t* new_slots,
                              const int32_t* req_to_token, int32_t table_rows, int64_t stride,
                              const int32_t* seq_lens, int32_t batch, const int32_t* plan_dev,
                              const rc_plan_info* info, float sm_scale, void* workspace,
                              int64_t ws_bytes, void* stream);

/* rc_decode_attention without a workspace argument, for callers that cannot */
/* allocate device memory (code under HIP graph capture, tight serving       */
/* loops, harnesses that forbid hipMalloc).  The partials go to a static     */
/* workspace inside the library: one array of                                */
/* RC_DECODE_STATIC_WORKSPACE_BYTES per GPU, created with the library's code */
/* on that GPU and held until the process ends.  A plan whose               */
/* rc_decode_workspace_bytes exceeds it fails with RC_ERR_RANGE before       */
/* anything is launched.  The call allocates nothing (no hipMalloc, no       */
/* events: kernel timing skips it); the first call on a device looks up the  */
/* array's address there (RC_ERR_HIP if that fails).  All calls on one GPU   */
/* share the array, whose contents persist from call to call (every partial  */
/* is written before it is read, so nothing needs clearing): calls that may  */
/* overlap on one GPU (other streams, other threads) race and give wrong     */
/* results; serialise them.  Arguments, outputs and errors otherwise as      */
/* rc_decode_attention.                                                      */
#define RC_DECODE_STATIC_WORKSPACE_BYTES (64ll << 20)
rc_status rc_decode_attention_static(const rc_shape* shape, void* o, const void* q, void* k_pool, void* v_pool,
                                     const void* k_new, const void* v_new, const int32_t* new_slots,
                                     const int32_t* req_to_token, int32_t table_rows, int64_t stride,
                                     const int32_t* seq_lens, int32_t batch, const int32_t* plan_dev,
                                     const rc_plan_info* info, float sm_scale, void* stream);

/* ------------------------------------------------------------------------ */
/* Radix tree over token ids, with the KV-pool slot allocator  ([SG]         */
/* RadixAttention bullet and nine-step example; [PC] exact-prefix reuse).    */
/* Host only; a handle is not thread-safe, separate handles are independent. */
/* Every call is atomic: on failure the tree and allocator are unchanged.    */
/* ------------------------------------------------------------------------ */
typedef struct rc_radix rc_radix;

typedef struct rc_radix_stats {
  int64_t nodes;           /* live nodes, root excluded                        */
  int64_t cached_tokens;   /* tokens held by the tree                          */
  int64_t free_slots;
  int64_t pool_slots;
  int64_t splits;          /* edge splits so far                               */
  int64_t matches;         /* match calls (including those inside emit_rows)   */
  int64_t matched_tokens;  /* sum of matched lengths                           */
  int64_t inserted_tokens; /* tokens newly stored by insert                    */
  int64_t duplicate_slots; /* slots freed because their prefix was already stored */
  int64_t evicted_tokens;  /* tokens removed by LRU eviction                   */
  int64_t evicted_nodes;
  int64_t locked_tokens;   /* tokens in nodes pinned by at least one lock       */
  int64_t page_symbols;    /* paged tree: distinct page contents it holds (each */
                           /* freed with its last holder); 0 when unpaged       */
} rc_radix_stats;

/* free_order (host, nullable): the initial order in which slots are handed   */
/* out, a permutation of [0, pool_slots); NULL means 0, 1, 2, ...            */
rc_status rc_radix_create(int64_t pool_slots, const int32_t* free_order, rc_radix** out);

/* A paged tree ("Prompt Caching" glossary, serving engines: KV kept in       */
/* fixed-size blocks, the blocks of the longest matching prefix reused): the  */
/* pool is n_pages pages of page_size (a power of two up to 1024) consecutive */
/* slots, the same page size as rc_shape.page_size.  Every call below takes   */
/* token ids as usual, but the tree stores, matches and shares whole pages:   */
/* only the full pages of a sequence are inserted, a prefix matches in whole  */
/* pages (a partly matching page is computed again), and "slots" are page ids */
/* everywhere (alloc, free, evict, the rows of req_to_token, whose stride     */
/* counts pages).  In detail:                                                 */
/*   match      at most (n - 1) / page_size pages; *matched in tokens;        */
/*              out_slots gets the matched page ids.                           */
/*   insert     stores the n / page_size full pages; slots_inout holds their  */
/*              page ids; n_new counts pages.                                  */
/*   emit_rows  row b gets ceil((n_b + reserve) / page_size) page ids:        */
/*              [matched pages | fresh pages]; prefix_lens = matched pages x  */
/*              page_size, extend_lens = n_b - prefix_lens (tokens).          */
/*   insert_rows, fork, lock: whole pages of the given tokens; lock's         */
/*              *locked in tokens.                                             */
/*   plan_decode, plan_extend: positions in tokens, as for unpaged trees.     */
/*   stats      token counts are in pages.                                     */
/* free_order (nullable) is a permutation of [0, n_pages).                     */
rc_status rc_radix_create_paged(int64_t n_pages, int32_t page_size, const int32_t* free_order, rc_radix** out);
void rc_radix_destroy(rc_radix* tree);

/* Longest cached prefix of tokens[0..n), capped at n-1 (a request always     */
/* runs at least one token).  out_slots (host, capacity n, nullable) gets    */
/* the slots of the matched tokens.  Marks every node that tokens[0..n)     */
/* enter (at least one token matched) as used now.                           */
rc_status rc_radix_match(rc_radix* tree, const int32_t* tokens, int64_t n, int32_t* out_slots,
                         int64_t* matched);

/* Take n slots first-in first-out from the free list (all or nothing).      */
rc_status rc_radix_alloc(rc_radix* tree, int64_t n, int32_t* out_slots);

/* Return slots to the back of the free list.  Slots already free, out of    */
/* range or repeated are rejected (RC_ERR_ARG) and nothing is freed.         */
rc_status rc_radix_free(rc_radix* tree, const int32_t* slots, int64_t n);

/* Store tokens[0..n) with their slots.  An edge is split at the first       */
/* divergence.  Where a prefix is already stored its stored slots win: the   */
/* caller's different slots for those positions are freed (ascending         */
/* position order) and slots_inout is overwritten with the stored ones, so   */
/* the caller can rewrite its table row.  n_new (nullable): tokens stored.   */
/* Marks as used now the nodes the tokens pass through and the new leaf; of  */
/* a split edge only the upper part (the part the tokens matched).           */
rc_status rc_radix_insert(rc_radix* tree, const int32_t* tokens, int32_t* slots_inout, int64_t n,
                          int64_t* n_new);

/* Token batches (host, CSR): request b owns tokens[tok_off[b] ..          */
/* tok_off[b+1]).  Where a call takes tok_len (nullable) only the first      */
/* tok_len[b] of them are used (0 <= tok_len[b] <= its count, else          */
/* RC_ERR_ARG), so one flattened batch serves schedule, commit and plan.     */

/* Batched insert ("commit"): for each request b, rc_radix_insert of its     */
/* tokens with the slots held in row rows[b] of the host table, rewriting    */
/* that row in place where the tree already held the tokens.  changed (host, */
/* nullable, batch entries) is set to 1 for rows that were rewritten.        */
/* Requests are processed in order; on a failure the requests before the     */
/* failing one stay inserted (RC_ERR_* names it).                            */
rc_status rc_radix_insert_rows(rc_radix* tree, int32_t batch, const int32_t* tokens, const int64_t* tok_off,
                               const int64_t* tok_len, const int32_t* rows, int32_t* req_to_token,
                               int32_t table_rows, int64_t stride, int32_t* changed);

/* Rows of the request -> slot table for a batch.  Request b has tokens      */
/* tokens[tok_off[b] .. tok_off[b+1]) (host, CSR).  Row rows[b] of the host   */
/* table req_to_token [*, stride] receives [matched prefix slots | new slots */
/* for the n_b - P_b uncached tokens | `reserve` more slots for decoding];   */
/* prefix_lens[b] = P_b, extend_lens[b] = n_b - P_b.  Allocation for the     */
/* whole batch is all or nothing, in request order.  Entries after the row's */
/* end are not touched.  table_rows bounds rows[b]; each row must fit in     */
/* stride (n_b + reserve <= stride) or the call fails with RC_ERR_RANGE.     */
/* Every node the requests' tokens enter is marked as used now (one time     */
/* for the whole batch).                                                     */
/*   flags     RC_EMIT_EVICT: when too few slots are free, first free the    */
/*             missing ones by rc_radix_evict (the batch's matched prefixes  */
/*             are pinned meanwhile, so the rows still get them); if that is */
/*             not enough the call fails with RC_ERR_NOMEM, the rows and     */
/*             locks untouched, but what was evicted and the use marks stay. */
/*             Without it too few free slots fail with RC_ERR_NOMEM and      */
/*             change nothing.                                               */
/*             RC_EMIT_FULL_MATCH: the match is not capped at n_b - 1, so a  */
/*             fully cached request gets E_b = 0 (for storing K/V computed  */
/*             elsewhere, not for running the request).  Other bits:         */
/*             RC_ERR_ARG.                                                    */
/*   handles (host, nullable, batch entries): also lock each request's       */
/*             matched prefix (as rc_radix_lock of its first P_b tokens) and */
/*             return the handles; release them with rc_radix_unlock.        */
/*   first_changed (host, nullable, batch entries): index of the first entry */
/*             of row rows[b] whose value this call changed (the row's entry */
/*             count if none did).  Entries before it hold what they held    */
/*             before the call, so a caller that mirrors the table on the    */
/*             device uploads only [first_changed[b], row entries).           */
/*   row_entries (host, nullable, batch entries): the entries row rows[b]    */
/*             now uses, n_b + reserve (tokens) or ceil((n_b + reserve) /    */
/*             page_size) (paged tree).                                      */
/*   new_slots (host, nullable, room for sum_b n_b entries): the pool slots  */
/*             of the new tokens, request after request: positions P_b ..    */
/*             n_b - 1 of request b at offset sum_{c<b} E_c; in a paged tree */
/*             position p's slot is page(p / page_size) * page_size +        */
/*             p % page_size.  These are the slots rc_kv_store fills.         */
#define RC_EMIT_EVICT 1
#define RC_EMIT_FULL_MATCH 2
rc_status rc_radix_emit_rows(rc_radix* tree, int32_t batch, const int32_t* tokens,
                             const int64_t* tok_off, int32_t reserve, const int32_t* rows,
                             int32_t* req_to_token, int32_t table_rows, int64_t stride,
                             int32_t* prefix_lens, int32_t* extend_lens, int32_t flags,
                             int64_t* handles, int64_t* first_changed, int64_t* row_entries,
                             int32_t* new_slots);

/* Return a batch's own slots when its requests end: for each request b,    */
/* the units (slots, or pages in a paged tree) of row rows[b] of the host    */
/* table from entry keep_lens[b] / page_size up to row_entries[b]: the       */
/* positions from its first token not kept in the tree (a partly kept page   */
/* is never in the tree) to the end of its row.  keep_lens in tokens,        */
/* row_entries as rc_radix_emit_rows reported them.  All or nothing, with   */
/* rc_radix_free's checks (a unit already free or given twice: RC_ERR_ARG).  */
rc_status rc_radix_free_rows(rc_radix* tree, int32_t batch, const int32_t* rows, const int32_t* req_to_token,
                             int32_t table_rows, int64_t stride, const int64_t* keep_lens,
                             const int64_t* row_entries);

/* Locks and LRU eviction ([SG] RadixAttention bullet: an LRU cache of KV in */
/* the radix tree; nine-step example, steps 5, 8 and 9: least recently used  */
/* nodes are evicted when memory runs short, never the ones a running        */
/* request reads).                                                           */
/* rc_radix_lock: for each request b, pin the nodes holding the cached       */
/* prefix of its first tok_len[b] tokens (all with tok_len NULL): the        */
/* deepest node entered and all its ancestors, that whole node included      */
/* even when the prefix ends inside its edge.  handles[b] (host) receives a  */
/* handle (0 when nothing is cached: nothing pinned), locked[b] (nullable)   */
/* the cached length.  A pinned node is never evicted; when its edge is      */
/* split later both parts stay pinned.  Locks do not mark nodes as used.     */
rc_status rc_radix_lock(rc_radix* tree, int32_t batch, const int32_t* tokens, const int64_t* tok_off,
                        const int64_t* tok_len, int64_t* handles, int64_t* locked);

/* Release n locks (handles from rc_radix_lock or rc_radix_emit_rows; 0 is a */
/* no-op).  Each lock is released once; a handle whose node no longer exists */
/* or whose counts are not held fails with RC_ERR_ARG and nothing changes.   */
rc_status rc_radix_unlock(rc_radix* tree, const int64_t* handles, int32_t n);

/* Free at least n_slots slots by evicting whole nodes: repeatedly the leaf  */
/* that no lock pins with the oldest last use (ties: the lower first slot of */
/* its edge); its slots go to the back of the free list in position order,   */
/* and a parent left without children becomes a candidate.  Stops early when */
/* nothing is evictable; freed (nullable) gets the number of slots freed.    */
/* n_slots <= 0 evicts nothing.                                              */
rc_status rc_radix_evict(rc_radix* tree, int64_t n_slots, int64_t* freed);

/* fork ([SG] primitive list: parallel copies of a prompt state): store the  */
/* parent's first n tokens with their slots (parent_slots, from its row) and */
/* copy those n slots into rows child_rows[0..n_children) of req_to_token.   */
/* The children then extend from the shared prefix without copying KV.       */
rc_status rc_radix_fork(rc_radix* tree, const int32_t* tokens, const int32_t* parent_slots, int64_t n,
                        int32_t n_children, const int32_t* child_rows, int32_t* req_to_token,
                        int32_t table_rows, int64_t stride);

/* Shared decode plan from the tree: request b's committed tokens (its      */
/* tok_len[b] first, or all) are walked through the tree; every node         */
/* range is one item whose members are all batch requests passing through    */
/* it (split into items of at most max(1, RC_DECODE_COLS / group) members);*/
/* positions                                                                 */
/* past the walked prefix up to max_seq_lens[b] form the request's own tail. */
/* A range is cut into the fewest near-equal pieces of at most chunk +      */
/* chunk/8 positions.  Table rows must                                        */
/* hold the tree's slots over the walked prefix (emit_rows + insert give     */
/* that).  Output as rc_plan_decode_unshared.                                */
rc_status rc_radix_plan_decode(rc_radix* tree, int32_t batch, const int32_t* tokens,
                               const int64_t* tok_off, const int64_t* tok_len, const int32_t* rows,
                               const int32_t* max_seq_lens, int32_t group, int32_t chunk,
                               int32_t* plan, int64_t capacity, rc_plan_info* info);

/* Shared-prefix ("cascade") extend plan.  The members of this plan are the  */
/* batch's new tokens, in batch order (member m = loc_b + i for token i of   */
/* request b, the same index as in q/o of rc_extend_attention).  Request b   */
/* has tokens tokens[tok_off[b] .. tok_off[b+1]) (host, CSR), of which the   */
/* first prefix_lens[b] are cached in the tree and the next extend_lens[b]   */
/* are new (their K/V already stored in their slots).  Token i of request b  */
/* attends over positions [0, prefix_lens[b] + i] of table row rows[b]        */
/* (NULL rows: b): the attention is the extend's (the SGLang summary's       */
/* RadixAttention over a shared prompt, "Prompt Caching" glossary, new       */
/* tokens over the cached prefix) computed as split-K decode over the plan:  */
/* every tree range on the prefixes is read once for all the new tokens      */
/* that pass through it (e.g. 64 label branches of one document read the     */
/* document once per group of RC_EXTEND_SHARED_COLS / group tokens, not      */
/* once per branch), and                                                     */
/* each token reads its own request's new tokens up to itself alone.        */
/* Run it with rc_extend_attention_shared.  Output and sizing as            */
/* rc_plan_decode_unshared; RC_ERR_RANGE also when a request's prefix +      */
/* extend exceed its tokens.  seq_lens (host, nullable, one entry per new    */
/* token) receives each token's context length prefix_lens[b] + i + 1, the  */
/* seq_lens rc_extend_attention_shared takes (written on success only).     */
rc_status rc_radix_plan_extend(rc_radix* tree, int32_t batch, const int32_t* tokens, const int64_t* tok_off,
                               const int32_t* prefix_lens, const int32_t* extend_lens, const int32_t* rows,
                               int32_t group, int32_t chunk, int32_t* plan, int64_t capacity,
                               rc_plan_info* info, int32_t* seq_lens);

/* Extend attention over a shared-prefix plan (rc_radix_plan_extend): the    */
/* same outputs as rc_extend_attention, o[m] for new token m (token i of     */
/* request b) = softmax attention of q[m] over positions [0, seq_lens[m])    */
/* of its request's table row, computed by the split-K kernels and the       */
/* merge of rc_decode_attention (the kernels are the decode kernels; their   */
/* launches are named extend_shared_* in profiles).                          */
/*   o, q      device [n_tokens, Hq, D] (shape dtype); q is read only.       */
/*   k_pool, v_pool  device [pool_slots, Hkv, D]: every key, the new tokens' */
/*             own included, is read from the pool, so store the new K/V    */
/*             first (rc_kv_store).                                          */
/*   seq_lens  device int32 [n_tokens]: prefix_lens[b] + i + 1.              */
/*   plan_dev / info / workspace: as rc_decode_attention (workspace size     */
/*             from rc_decode_workspace_bytes of this plan).                 */
/* Errors as rc_decode_attention; info->batch must equal n_tokens.           */
rc_status rc_extend_attention_shared(const rc_shape* shape, void* o, const void* q, const void* k_pool,
                                     const void* v_pool, const int32_t* req_to_token, int32_t table_rows,
                                     int64_t stride, const int32_t* seq_lens, int32_t n_tokens,
                                     const int32_t* plan_dev, const rc_plan_info* info, float sm_scale,
                                     void* workspace, int64_t ws_bytes, void* stream);

rc_status rc_radix_stats_get(const rc_radix* tree, rc_radix_stats* out);

/* ------------------------------------------------------------------------ */
/* Label-restricted next-token distribution for single-token classification */
/* (openjev-sglang tutorial: "how inference works", step 5, the question     */
/* types and "interpret confidence carefully").  For row r of logits (the   */
/* next-token logits after a branch, e.g. the classification branches of    */
/* one document) with k_r = counts[r] options (all n_labels when counts is  */
/* NULL), over the first k_r label tokens label_ids[0..k_r):                 */
/*   probs[r, i]   = exp(x_i - max x) / sum_j exp(x_j - max x), x_i =        */
/*                   logits[r, label_ids[i]] (stable softmax), 0 for i >= k_r */
/*   choice[r]     = the option with the largest logit (lowest index on ties) */
/*   expected[r]   = sum_i i * probs[r, i] (the Score question's expected     */
/*                   zero-based level)                                       */
/*   confidence[r] = 1 - H(probs[r]) / log(k_r), natural log, 0 log 0 = 0;  */
/*                   1 when k_r = 1                                          */
/* A Bool question is the two-option case with the labels (yes, no): its    */
/* answer is probs[r, 0].                                                    */
/*   logits     device [n_rows, row_stride] of dtype (RC_F32 or RC_BF16),     */
/*              finite; only the first vocab entries of a row are read.     */
/*   label_ids  device int32 [n_labels], 1 <= n_labels <= 64, each in        */
/*              [0, vocab) (else RC_DEVERR_LABEL and the label gets          */
/*              probability 0).                                              */
/*   counts     device int32 [n_rows] or NULL; out-of-range counts are       */
/*              clamped into [1, n_labels] and raise RC_DEVERR_LABEL.        */
/*   probs      device float [n_rows, n_labels]; choice (int32), expected,   */
/*              confidence (float): device [n_rows], each nullable.          */
/* fp32 arithmetic; deterministic (fixed reduction order).                   */
rc_status rc_label_distribution(const void* logits, int32_t dtype, int64_t row_stride, int64_t vocab,
                                int32_t n_rows, const int32_t* label_ids, int32_t n_labels,
                                const int32_t* counts, float* probs, int32_t* choice, float* expected,
                                float* confidence, void* stream);

/* ------------------------------------------------------------------------ */
/* Kernel timing.  While enabled, every kernel the library launches is       */
/* bracketed by HIP events on its own stream.  rc_prof_collect waits for the */
/* recorded events, returns per-kernel totals and clears them.  Enabling     */
/* creates a pool of events up front (16384 with those already recorded), so*/
/* timed launches only record them; RC_ERR_HIP if creating one fails.       */
/* ------------------------------------------------------------------------ */
typedef struct rc_prof_entry {
  char name[48];
  int64_t launches;
  double total_ms;
} rc_prof_entry;

rc_status rc_prof_enable(int32_t on);
/* Launches timed after this call are reported as "<kernel>@<tag>" (tag cut  */
/* to 15 characters; NULL or "" for the plain kernel name), so one kernel's  */
/* launches in different phases of a step are told apart.                    */
rc_status rc_prof_tag(const char* tag);
rc_status rc_prof_collect(rc_prof_entry* out, int32_t capacity, int32_t* n_out);

#ifdef __cplusplus
}
#endif
#endif /* RC_H */
