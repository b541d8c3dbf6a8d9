/*
 * pkv.h -- C ABI of libpkv.so: paged KV-cache decode attention for gfx950.
 *
 * Sources (the three pages on LLM-inference optimisation this library
 * follows; cited by key and section):
 *   hotelren = www.hotelren.com/news/4669576
 *   dpshk    = www.dpshk.com/news/5622214
 *   pgsm     = www.pgsm.cn/news/396587
 *              (LLM推理优化：从硬件瓶颈到KV Cache的工程实践)
 *
 * Data layout shared by every device entry point
 * ----------------------------------------------
 *   K pool, V pool : fp16 storage of shape [N][Hkv][P / 16][16 * D]: N pages
 *                    x Hkv KV heads x P / 16 sub-blocks of 16 tokens, each
 *                    sub-block 16 * D halves; the P * D halves of a (page, KV
 *                    head) tile are contiguous. A page holds P tokens of
 *                    every KV head (hotelren §3.2 and pgsm §3.2 describe a
 *                    page as tokens x heads x dims in fp16; the order inside a
 *                    tile is this library's choice). The storage is NOT a
 *                    [token][dim] array: token u = t % 16 of sub-block t / 16,
 *                    dim d, sits at
 *                      K: ((d / 8) * 16 + u) * 8 + d % 8
 *                      V: (((d / 32) * 4 + u / 4) * 16 + d % 16) * 8
 *                         + ((d / 16) % 2) * 4 + u % 4
 *                    inside its sub-block, so that consecutive 16-byte runs are
 *                    the matrix-core operands of the decode kernel. Use
 *                    pkv_kv_append (or the same formulas) to write tokens.
 *   block table    : int32 [B][max_pages], row-major. Entry j of row b is the
 *                    physical page of logical tokens j*P .. j*P+P-1 of
 *                    sequence b (the page table of pgsm §3.2 and §4.1).
 *                    Unused entries may hold anything (the allocator writes -1).
 *   token t of sequence b is token t % P of page bt[b][t / P].
 *   query head h reads KV head h / (Hq / Hkv).
 *
 * Conventions
 * -----------
 *   - Every function returns a pkv_status (0 = PKV_OK). Nothing throws, aborts
 *     or keeps global error state.
 *   - Device pointers are caller-owned device memory. fp16 tensors must be
 *     16-byte aligned; int32 tensors 4-byte aligned. Nothing is allocated,
 *     freed or synchronised inside a device entry point: work is enqueued on
 *     `stream` (a hipStream_t; NULL is the default stream) and the call returns.
 *   - Argument checks run on the host before any launch; a failed check
 *     launches nothing. PKV_ERR_HIP is returned only when a launch fails.
 *   - Device-resident contents (block-table entries, lengths, positions) are
 *     not validated per call, which would need a synchronisation. Kernels never
 *     read or write outside the buffers described by the sizes passed in:
 *     a page id outside [0, N) or a length beyond the table width /
 *     max_context turns the affected output row into NaN, and an append whose
 *     slot is out of range is skipped. pkv_validate_tables checks host copies.
 *   - lens[b] == 0 marks an idle batch slot on every decode path: its output
 *     rows are zero, none of its pages is read and nothing is appended.
 *   - Supported: D in {64, 128}; P in {16, 32, 64, 128}; Hq / Hkv in
 *     {1, 2, 4, 8, 16}. Other values return PKV_ERR_UNSUPPORTED.
 */
#ifndef PKV_H_
#define PKV_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum pkv_status {
  PKV_OK = 0,
  PKV_ERR_INVALID_ARG = 1,          /* null/misaligned pointer, bad size or shape */
  PKV_ERR_UNSUPPORTED = 2,          /* valid but not built: D, P or group size */
  PKV_ERR_OUT_OF_PAGES = 3,         /* allocator cannot cover a reservation */
  PKV_ERR_WORKSPACE_TOO_SMALL = 4,  /* split decode given too little workspace */
  PKV_ERR_HIP = 5,                  /* a kernel launch failed */
  PKV_ERR_INVALID_TABLE = 6,        /* pkv_validate_tables found a bad entry */
  PKV_ERR_NOT_FOUND = 7,            /* pkv_alloc_cache_lookup: no entry under the key */
  PKV_ERR_HOST_MEMORY = 8,          /* the host allocator's own bookkeeping could not grow */
  PKV_ERR_SCRATCH_LIMIT = 9         /* a call needs more than the fixed scratch of the no-allocation entry */
} pkv_status;

/* Human-readable name of a status code (static string, never NULL). */
const char* pkv_status_string(int status);

/* ABI version of this header: 2. */
int pkv_abi_version(void);

/* ------------------------------------------------------------------------ */
/* Device entry points                                                      */
/* ------------------------------------------------------------------------ */

/*
 * pkv_block_table_patch -- set entries of a device block table from a short
 * host list, without a host-to-device copy.
 *
 * Decode grows the page table one page at a time as sequences cross page
 * boundaries (pages are taken on demand, dpshk §4.2; pgsm §4.3), so after a
 * step only a few entries differ from the device copy. The entries travel in
 * the kernel arguments of a one-workgroup launch (up to 128 per launch; longer
 * lists take several), so the update is ordered on `stream` like any kernel
 * and needs no staging buffer or DMA.
 *
 *   block_table : int32 [B][max_pages] device, written at the listed entries.
 *   rows, cols, pages: int32 [n] HOST arrays (read during the call; the
 *                 caller may reuse them on return): entry (rows[i], cols[i])
 *                 becomes pages[i]. List each entry at most once: two
 *                 writes of one entry in the same launch land in no set
 *                 order.
 * Errors: PKV_ERR_INVALID_ARG (n < 0, a row outside [0, B), a column outside
 * [0, max_pages), a page below -1, null pointers, misaligned table; nothing is
 * launched), PKV_ERR_HIP.
 */
int pkv_block_table_patch(int32_t* block_table, int32_t B, int32_t max_pages, const int32_t* rows,
                          const int32_t* cols, const int32_t* pages, int32_t n, void* stream);

/*
 * pkv_kv_append -- write each sequence's new-token K and V into its page slot.
 *
 * Decode appends the new token's K and V (one D-vector per KV head each) to
 * the cache and never recomputes older entries (pgsm §3.2 and §4.3); the write
 * goes in place into preallocated storage instead of growing a tensor
 * (hotelren §3.1, pgsm §4.3).
 *
 *   k_new, v_new : fp16 [B][Hkv][D] device, read.
 *   k_pool, v_pool: fp16 pools (layout above) device, written only at the
 *                  D halves of token pos[b] % P of page bt[b][pos[b] / P],
 *                  KV head kvh, for every b, kvh.
 *   block_table  : int32 [B][max_pages] device, read.
 *   pos          : int32 [B] device: position of the new token (the length
 *                  of the context before the append).
 * The copy is bit-exact. A position outside [0, max_pages * P) or a page id
 * outside [0, N) skips that sequence. B == 0 is a no-op.
 * Errors: PKV_ERR_INVALID_ARG, PKV_ERR_UNSUPPORTED, PKV_ERR_HIP.
 */
int pkv_kv_append(const void* k_new, const void* v_new, void* k_pool, void* v_pool,
                  const int32_t* block_table, int32_t max_pages, const int32_t* pos,
                  int32_t B, int32_t Hkv, int32_t D, int32_t P, int32_t N, void* stream);

/*
 * pkv_kv_append_chunk -- pkv_kv_append for n_tokens consecutive tokens per
 * sequence in one launch: the keys and values of a chunk (the drafted tokens
 * a verification step scores, or a prefill chunk; pgsm §3.2), written in
 * place like single tokens (pgsm §4.3).
 *
 *   k_new, v_new : fp16 [B][n_tokens][Hkv][D] device, read.
 *   pos          : int32 [B] device: token i of sequence b goes to position
 *                  pos[b] + i (every position must have its page in the
 *                  table; a position outside it, or a page id outside [0, N),
 *                  skips that token).
 *   n_tokens     : >= 1; n_tokens == 1 is pkv_kv_append.
 * Other arguments and errors as pkv_kv_append.
 */
int pkv_kv_append_chunk(const void* k_new, const void* v_new, void* k_pool, void* v_pool,
                        const int32_t* block_table, int32_t max_pages, const int32_t* pos, int32_t B,
                        int32_t n_tokens, int32_t Hkv, int32_t D, int32_t P, int32_t N, void* stream);

/*
 * pkv_decode_workspace_bytes -- workspace size split-context decode needs.
 *
 * In split mode the private tokens of every sequence are divided among a
 * fixed set of workgroups (see pkv_paged_decode_attention); each piece a
 * workgroup takes of a (sequence, KV head) leaves, per query head, a float
 * max, a float sum and D floats of unnormalised output, plus a small header
 * and one int per sequence. The size does not depend on max_context.
 * partition_tokens == 0 needs no workspace (*bytes = 0).
 * Errors: PKV_ERR_INVALID_ARG (negative sizes, partition_tokens not a
 * multiple of 16, B > 4096 with partition_tokens > 0, null `bytes`).
 * The size holds for every Hkv dividing Hq and every device.
 */
int pkv_decode_workspace_bytes(int32_t B, int32_t Hq, int32_t D, int32_t max_context,
                               int32_t partition_tokens, size_t* bytes);

/*
 * pkv_paged_decode_attention -- single-token decode attention through the
 * page table.
 *
 * For every sequence b and query head h: read the lens[b] cached keys and
 * values of KV head h / (Hq / Hkv) through the block table, score
 * s_t = scale * <q[b][h], k_t>, softmax over t, and write the weighted sum of
 * the values (pgsm §4.2 describes exactly these four steps of a decode step:
 * read all past KV, score, normalise, weighted sum). Accumulation is fp32
 * (dpshk §3.3 keeps high-precision accumulation on the critical path); the
 * result is rounded to fp16 (round to nearest even).
 *
 *   out          : fp16 [B][Hq][D] device, written.
 *   q            : fp16 [B][Hq][D] device, read.
 *   k_pool/v_pool: fp16 pools (layout above) device, read.
 *   block_table  : int32 [B][max_pages] device, read.
 *   lens         : int32 [B] device: tokens to attend (the new token
 *                  included). lens[b] == 0 writes a zero row.
 *   max_context  : host upper bound on every lens[b]; sizes the launch and
 *                  the workspace; must be <= max_pages * P.
 *   scale        : softmax scale, normally 1/sqrt(D); positive and finite
 *                  (else PKV_ERR_INVALID_ARG).
 *   partition_tokens: 0 = one workgroup per (sequence, KV head) over the whole
 *                  context, writing the output directly. Otherwise a positive
 *                  multiple of 16 (split mode, at most 4096 sequences): the
 *                  16-token blocks of all (KV head, sequence) contexts form
 *                  one list that is divided evenly among a fixed set of
 *                  workgroups (two per compute unit of the current device),
 *                  each taking at least partition_tokens tokens
 *                  (pieces may cross from one sequence into the next); a
 *                  log-sum-exp reduction kernel then merges the pieces of
 *                  every sequence. This balances batches of mixed lengths.
 *   workspace    : device buffer of at least pkv_decode_workspace_bytes bytes
 *                  (ignored when partition_tokens == 0), 256-byte aligned.
 * Errors: PKV_ERR_INVALID_ARG, PKV_ERR_UNSUPPORTED,
 * PKV_ERR_WORKSPACE_TOO_SMALL, PKV_ERR_HIP.
 */
int pkv_paged_decode_attention(void* out, const void* q, const void* k_pool, const void* v_pool,
                               const int32_t* block_table, int32_t max_pages, const int32_t* lens,
                               int32_t B, int32_t Hq, int32_t Hkv, int32_t D, int32_t P, int32_t N,
                               int32_t max_context, float scale, int32_t partition_tokens,
                               void* workspace, size_t workspace_bytes, void* stream);

/*
 * pkv_append_paged_decode_attention -- append then attend, in one launch.
 *
 * Same result as pkv_kv_append(k_new, v_new, ..., pos = lens - 1) followed by
 * pkv_paged_decode_attention(...): the new token is part of the context it
 * attends to (hotelren §3.1: write the new K/V at the end, then attend). The
 * wave that streams the block holding the new token takes its K/V from k_new /
 * v_new into registers and uses them there, saving a launch per step. The
 * pool write itself goes to the merge launch that follows in split mode
 * (stores issued while every compute unit streams reads cost microseconds)
 * and to the streaming wave when unsplit; either way it is done when the
 * call's work on the stream is.
 * lens[b] >= 1 is the context after the append; lens[b] == 0 writes a zero
 * row and appends nothing. Arguments as in the two calls above.
 */
int pkv_append_paged_decode_attention(void* out, const void* q, const void* k_new, const void* v_new,
                                      void* k_pool, void* v_pool, const int32_t* block_table,
                                      int32_t max_pages, const int32_t* lens, int32_t B, int32_t Hq,
                                      int32_t Hkv, int32_t D, int32_t P, int32_t N, int32_t max_context,
                                      float scale, int32_t partition_tokens, void* workspace,
                                      size_t workspace_bytes, void* stream);

/*
 * pkv_decode_workspace_bytes_shared_prefix -- workspace size for
 * pkv_paged_decode_attention_shared_prefix: the split path's per-sequence
 * block counts and per-piece partials (score max, denominator, D outputs for
 * 16 query rows), with one extra segment per 16 query rows of a KV head for
 * the shared prefix.
 * Errors: PKV_ERR_INVALID_ARG (as pkv_decode_workspace_bytes; prefix_tokens
 * negative, not a multiple of 16, above max_context, or > 0 with
 * partition_tokens == 0).
 */
int pkv_decode_workspace_bytes_shared_prefix(int32_t B, int32_t Hq, int32_t D, int32_t max_context,
                                             int32_t partition_tokens, int32_t prefix_tokens, size_t* bytes);

/*
 * pkv_decode_workspace_bytes_multi -- workspace size for the chunked calls
 * (pkv_paged_decode_attention_multi, _multi_shared_prefix, _multi_k8,
 * _window_multi, _window_multi_k8) with n_query queries per sequence: one
 * private segment per sequence and group of up to four 16-column query tiles
 * (chunks of pgsm §3.2's draft verification and chunked prefill), one prefix
 * segment per group of up to four 16-row tiles of a KV head's chunk rows when
 * prefix_tokens > 0. n_query == 1 gives the single-query sizes. Errors:
 * PKV_ERR_INVALID_ARG (as pkv_decode_workspace_bytes_shared_prefix;
 * n_query < 1; more than 4096 segments for every allowed Hkv).
 */
int pkv_decode_workspace_bytes_multi(int32_t B, int32_t n_query, int32_t Hq, int32_t D, int32_t max_context,
                                     int32_t partition_tokens, int32_t prefix_tokens, size_t* bytes);

/*
 * pkv_paged_decode_attention_shared_prefix -- decode for a batch whose
 * sequences all begin with the same prefix_tokens tokens held in the same
 * physical pages (a system prompt stored once and shared by every request:
 * dpshk §4.2, pgsm §3.2 and §4.3).
 *
 * Same result as pkv_paged_decode_attention (after the append, if k_new and
 * v_new are given), computed so that the shared pages are read once per KV
 * head and 16 query rows instead of once per sequence: the prefix blocks are
 * scored against 16 query rows of a KV head at a time (a full matrix-core
 * tile), and these prefix pieces and every sequence's private blocks form one
 * work list per KV head, cut evenly among the split path's workgroups; the
 * log-sum-exp reduction merges both.
 *
 *   prefix_tokens: multiple of P, 0 <= prefix_tokens <= max_context; entries
 *                  0 .. prefix_tokens / P - 1 must be identical in every
 *                  attended row (lens[b] > 0): they are read from the first
 *                  such row, and an idle row's entries are never read
 *                  (pkv_validate_tables with prefix_tokens checks this on host
 *                  copies). 0 < lens[b] < prefix_tokens makes row b NaN.
 *   k_new, v_new : both NULL (no append) or both fp16 [B][Hkv][D]: append
 *                  each sequence's new token at lens[b] - 1 first, as in
 *                  pkv_append_paged_decode_attention. That position must lie
 *                  after the prefix: with prefix_tokens > 0, a row with
 *                  lens[b] <= prefix_tokens is NaN and appends nothing.
 *   partition_tokens: > 0 (this path always splits).
 *   workspace    : at least pkv_decode_workspace_bytes_shared_prefix bytes.
 * Other arguments and errors as pkv_paged_decode_attention.
 */
int pkv_paged_decode_attention_shared_prefix(void* out, const void* q, const void* k_new, const void* v_new,
                                             void* k_pool, void* v_pool, const int32_t* block_table,
                                             int32_t max_pages, const int32_t* lens, int32_t B, int32_t Hq,
                                             int32_t Hkv, int32_t D, int32_t P, int32_t N, int32_t max_context,
                                             float scale, int32_t partition_tokens, int32_t prefix_tokens,
                                             void* workspace, size_t workspace_bytes, void* stream);

/*
 * pkv_paged_decode_attention_shared_prefix_noalloc -- for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc): pkv_paged_decode_attention_shared_prefix
 * without a workspace argument. The split path's partials and per-segment
 * prefix sums go to a fixed array of pkv_noalloc_scratch_bytes() (32 MiB)
 * that the library holds in every GPU it runs on until the process ends; its
 * device address is looked up on the first call on each device. The call
 * allocates nothing (no hipMalloc, no library allocation); the caller passes
 * the inputs and the output as for the workspace entry point, with the same
 * result bit for bit (same kernels, same schedule).
 * The array keeps the last call's contents; no part of it needs clearing
 * (every word a call reads was written earlier in the same call). Calls on
 * one GPU share the array, so calls that overlap in time on one GPU (other
 * streams, other host threads) race: order them on one stream.
 * Errors: as pkv_paged_decode_attention_shared_prefix, with
 * PKV_ERR_SCRATCH_LIMIT (nothing launched) when the split path needs more
 * than the fixed array (the Llama-3-8B GQA batch of 64 sequences needs about
 * 14 MB); PKV_ERR_HIP if the array's address cannot be found.
 */
int pkv_paged_decode_attention_shared_prefix_noalloc(void* out, const void* q, const void* k_new, const void* v_new,
                                                     void* k_pool, void* v_pool, const int32_t* block_table,
                                                     int32_t max_pages, const int32_t* lens, int32_t B, int32_t Hq,
                                                     int32_t Hkv, int32_t D, int32_t P, int32_t N,
                                                     int32_t max_context, float scale, int32_t partition_tokens,
                                                     int32_t prefix_tokens, void* stream);

/* Bytes of the fixed scratch array of the no-allocation entry point. */
size_t pkv_noalloc_scratch_bytes(void);

/*
 * pkv_paged_decode_attention_multi -- attention for a chunk of the last
 * n_query tokens of every sequence at once, causal within the chunk: the
 * verification of drafted tokens in speculative decoding, or one chunk of a
 * chunked prefill, over the same paged cache (pgsm §3.2 names both).
 *
 * Query i (0 <= i < n_query) of sequence b sits at position
 * lens[b] - n_query + i and attends tokens 0 .. lens[b] - n_query + i: each
 * query gets exactly the single-token decode of its own prefix. The chunk's
 * keys and values must already be in the cache (pkv_kv_append per token).
 *
 *   out          : fp16 [B][n_query][Hq][D] device, written.
 *   q            : fp16 [B][n_query][Hq][D] device, read.
 *   n_query      : >= 1. The n_query * (Hq / Hkv) query rows of a (sequence,
 *                  KV head) are cut into 16-column matrix-core tiles of 16 /
 *                  (Hq / Hkv) consecutive queries, and the tiles into groups
 *                  of up to four; the waves of a group's tiles stream the
 *                  sequence's tokens up to the group's last query together
 *                  (one read from memory, the others from the L2). In split
 *                  mode B * ceil(ceil(n_query * (Hq / Hkv) / 16) / 4) <= 4096.
 *   lens[b]      : tokens in the cache including the whole chunk; a row with
 *                  0 < lens[b] < n_query (or beyond max_context / the table)
 *                  is NaN; lens[b] == 0 gives zero rows.
 *   workspace    : pkv_decode_workspace_bytes_multi bytes.
 * Other arguments and errors as pkv_paged_decode_attention.
 */
int pkv_paged_decode_attention_multi(void* out, const void* q, const void* k_pool, const void* v_pool,
                                     const int32_t* block_table, int32_t max_pages, const int32_t* lens, int32_t B,
                                     int32_t n_query, int32_t Hq, int32_t Hkv, int32_t D, int32_t P, int32_t N,
                                     int32_t max_context, float scale, int32_t partition_tokens, void* workspace,
                                     size_t workspace_bytes, void* stream);

/*
 * pkv_paged_decode_attention_window -- decode over the last `window` tokens
 * of every sequence, its pages kept in a ring: the fixed-capacity cache that
 * overwrites its oldest entries (hotelren §3.2), through the page table.
 *
 * Sequence b owns ring_pages pages, row b of ring_table; its logical page j
 * (tokens j * P .. j * P + P - 1) lives in page ring_table[b][j % ring_pages],
 * so a new page overwrites the one ring_pages pages older. Query b attends
 * tokens max(0, lens[b] - window) .. lens[b] - 1 only, with softmax, scaling
 * and layout as in pkv_paged_decode_attention; token t is slot t % P of page
 * ring_table[b][(t / P) % ring_pages]. Pages of the ring that the window does
 * not reach are never read; slots of a reached page that lie before the window
 * are read and masked (their values never reach the output, NaN included).
 *
 *   ring_table   : int32 [B][ring_pages] device, read; every entry the window
 *                  reaches must be in [0, N) (else the row is NaN).
 *   ring_pages   : >= 1; window <= (ring_pages - 1) * P + 1, so that the pages
 *                  a window touches are distinct ring entries.
 *   lens[b]      : tokens of the sequence so far (any length up to
 *                  2^31 - 65; negative or longer makes the row NaN); 0 gives a
 *                  zero row.
 *   window       : >= 1 tokens attended.
 *   k_new, v_new : both NULL, or both fp16 [B][Hkv][D]: append each
 *                  sequence's new token at position lens[b] - 1 (into its
 *                  ring page) in the same launch, as
 *                  pkv_append_paged_decode_attention does.
 *   partition_tokens: 0 = one workgroup per (sequence, KV head); > 0 = the
 *                  split path over the window's blocks, workspace from
 *                  pkv_decode_workspace_bytes(B, Hq, D, window,
 *                  partition_tokens, ...).
 * Other arguments as pkv_paged_decode_attention.
 * Errors: PKV_ERR_INVALID_ARG (window <= 0, ring_pages <= 0, a window that
 * does not fit the ring, k_new without v_new, and the checks of
 * pkv_paged_decode_attention); PKV_ERR_UNSUPPORTED, PKV_ERR_WORKSPACE_TOO_SMALL
 * and PKV_ERR_HIP as there.
 */
int pkv_paged_decode_attention_window(void* out, const void* q, const void* k_new, const void* v_new, void* k_pool,
                                      void* v_pool, const int32_t* ring_table, int32_t ring_pages, const int32_t* lens,
                                      int32_t B, int32_t Hq, int32_t Hkv, int32_t D, int32_t P, int32_t N,
                                      int32_t window, float scale, int32_t partition_tokens, void* workspace,
                                      size_t workspace_bytes, void* stream);

/*
 * pkv_paged_decode_attention_window_multi -- chunks of queries (as
 * pkv_paged_decode_attention_multi: query i of sequence b at position
 * p = lens[b] - n_query + i) over a sliding window in a ring of pages (as
 * pkv_paged_decode_attention_window): query i attends the last `window`
 * tokens ending at itself, max(0, p + 1 - window) .. p. Drafted tokens of a
 * sliding-window model verified in one call; their keys and values must be in
 * the ring already (pkv_kv_append_chunk through the ring table's logical
 * pages).
 *
 *   q, out       : fp16 [B][n_query][Hq][D] device.
 *   ring_pages   : window + n_query - 1 <= (ring_pages - 1) * P + 1, so that
 *                  every token the chunk's windows reach is still in the ring.
 *   lens[b]      : tokens so far, the chunk included; 0 < lens[b] < n_query
 *                  (or negative, or above 2^31 - 65) makes the row NaN.
 *   workspace    : pkv_decode_workspace_bytes_multi(B, n_query, Hq, D, window,
 *                  partition_tokens, 0, ...) bytes when partition_tokens > 0.
 * Query tiles as in pkv_paged_decode_attention_multi. Errors as
 * pkv_paged_decode_attention_window and pkv_paged_decode_attention_multi.
 */
int pkv_paged_decode_attention_window_multi(void* out, const void* q, const void* k_pool, const void* v_pool,
                                            const int32_t* ring_table, int32_t ring_pages, const int32_t* lens,
                                            int32_t B, int32_t n_query, int32_t Hq, int32_t Hkv, int32_t D, int32_t P,
                                            int32_t N, int32_t window, float scale, int32_t partition_tokens,
                                            void* workspace, size_t workspace_bytes, void* stream);

/*
 * pkv_paged_decode_attention_multi_shared_prefix -- the chunked attention of
 * pkv_paged_decode_attention_multi for a batch whose sequences all begin with
 * the same prefix_tokens tokens in the same pages (drafted tokens verified
 * against a shared system prompt; pgsm §3.2 names both the chunks and prefix
 * reuse).
 *
 * Same result as pkv_paged_decode_attention_multi. The shared pages are read
 * as in pkv_paged_decode_attention_shared_prefix: once per KV head and 16
 * query rows, the rows now being the n_query * (Hq / Hkv) chunk rows of every
 * sequence. Every prefix token precedes every query of a chunk, so the prefix
 * needs no causal mask.
 *
 *   prefix_tokens: as in pkv_paged_decode_attention_shared_prefix; a row with
 *                  0 < lens[b] < prefix_tokens + n_query (a chunk reaching
 *                  into the prefix) is NaN.
 *   partition_tokens: > 0 (this path always splits).
 *   workspace    : at least pkv_decode_workspace_bytes_multi(B, n_query, Hq,
 *                  D, max_context, partition_tokens, prefix_tokens) bytes.
 * Other arguments and errors as pkv_paged_decode_attention_multi.
 */
int pkv_paged_decode_attention_multi_shared_prefix(void* out, const void* q, const void* k_pool, const void* v_pool,
                                                   const int32_t* block_table, int32_t max_pages, const int32_t* lens,
                                                   int32_t B, int32_t n_query, int32_t Hq, int32_t Hkv, int32_t D,
                                                   int32_t P, int32_t N, int32_t max_context, float scale,
                                                   int32_t partition_tokens, int32_t prefix_tokens, void* workspace,
                                                   size_t workspace_bytes, void* stream);

/* ------------------------------------------------------------------------ */
/* Key-only int8 pages                                                       */
/* ------------------------------------------------------------------------ */
/*
 * Keys quantised to int8, values kept fp16: quantising the KV cache halves
 * its memory but costs attention precision on long sequences, so the pages
 * advise quantising the keys only (dpshk §4.4), block-wise (pgsm §4.2). Here a
 * block is one token's D keys of one KV head, with its own fp32 scale: appends
 * never rewrite older tokens (pgsm §4.3), so a page-wide scale would have to
 * clip later tokens. Per token and KV head: scale = amax / 127 and
 * code = rint(k * (127 / amax)) (IEEE fp32, half to even; amax == 0 gives scale 0,
 * codes 0); the dequantised key is code * scale.
 *
 * int8-key pool: bytes [N][Hkv][P / 16][16 * D + 64]. A 16-token sub-block holds
 * the 16 x D codes, then the 16 fp32 scales (token u at byte 16 * D + 4 u).
 * The code of token u, dim d is at byte
 *   ((d / 64) * 64 + ((d / 8) % 4) * 16 + u) * 16 + ((d / 32) % 2) * 8 + d % 8,
 * so each 16-byte run holds one lane's matrix-core operand bytes for 64 dims.
 * The V pool is the fp16 pool described above. K bytes per token and head:
 * D + 4 instead of 2 D.
 * Supported: D in {64, 128}, P in {16, 32, 64, 128}, Hq / Hkv in {1..16}.
 */

/* pkv_k8_pool_bytes -- size of an int8-key pool. Errors: PKV_ERR_INVALID_ARG
 * (null bytes, N < 0, Hkv <= 0), PKV_ERR_UNSUPPORTED (D or P). */
int pkv_k8_pool_bytes(int32_t N, int32_t Hkv, int32_t P, int32_t D, size_t* bytes);

/*
 * pkv_kv_append_k8 -- as pkv_kv_append, with the key quantised into the
 * int8-key pool (codes and scale of the one token written) and the value into
 * the fp16 V pool. A position outside [0, max_pages * P) or a page id outside
 * [0, N) skips that sequence. Errors as pkv_kv_append.
 */
int pkv_kv_append_k8(const void* k_new, const void* v_new, void* k_pool8, void* v_pool, const int32_t* block_table,
                     int32_t max_pages, const int32_t* pos, int32_t B, int32_t Hkv, int32_t D, int32_t P, int32_t N,
                     void* stream);

/*
 * pkv_kv_append_k8_chunk -- pkv_kv_append_k8 for n_tokens consecutive tokens
 * per sequence in one launch (k_new, v_new fp16 [B][n_tokens][Hkv][D]; token
 * i of sequence b goes to position pos[b] + i), each key quantised on its
 * own as in pkv_kv_append_k8. Positions outside the table and page ids
 * outside [0, N) skip that token. Other arguments and errors as
 * pkv_kv_append_k8; n_tokens >= 1.
 */
int pkv_kv_append_k8_chunk(const void* k_new, const void* v_new, void* k_pool8, void* v_pool,
                           const int32_t* block_table, int32_t max_pages, const int32_t* pos, int32_t B,
                           int32_t n_tokens, int32_t Hkv, int32_t D, int32_t P, int32_t N, void* stream);

/*
 * pkv_paged_decode_attention_k8 -- pkv_paged_decode_attention_shared_prefix
 * (prefix_tokens == 0: no shared prefix, and then partition_tokens may be 0)
 * over int8 keys: s_t = scale * scale_t * <q, code_t>, the rest as for fp16
 * keys (fp32 accumulation, fp16 output).
 *   k_new, v_new : both NULL (no append) or both fp16 [B][Hkv][D]: append each
 *                  sequence's new token at lens[b] - 1 first, in the same
 *                  launch. The key is quantised exactly as pkv_kv_append_k8
 *                  does (same codes, same scale, bit for bit), written to the
 *                  pool and used from registers.
 * Workspace: pkv_decode_workspace_bytes / pkv_decode_workspace_bytes_shared_prefix.
 * Errors as pkv_paged_decode_attention_shared_prefix.
 */
int pkv_paged_decode_attention_k8(void* out, const void* q, const void* k_new, const void* v_new, void* k_pool8,
                                  void* v_pool, const int32_t* block_table, int32_t max_pages, const int32_t* lens,
                                  int32_t B, int32_t Hq, int32_t Hkv, int32_t D, int32_t P, int32_t N,
                                  int32_t max_context, float scale, int32_t partition_tokens, int32_t prefix_tokens,
                                  void* workspace, size_t workspace_bytes, void* stream);

/*
 * pkv_paged_decode_attention_multi_k8 -- chunks of queries (as
 * pkv_paged_decode_attention_multi: query i of sequence b at position
 * lens[b] - n_query + i, causal within the chunk) over int8-key pages: the
 * attention of verifying drafted tokens against a quantised cache. The
 * chunk's keys and values must be in the pools already
 * (pkv_kv_append_k8_chunk). prefix_tokens > 0 reads a shared prefix as
 * pkv_paged_decode_attention_multi_shared_prefix does. Workspace:
 * pkv_decode_workspace_bytes_multi(B, n_query, ..., prefix_tokens). Other
 * arguments and errors as pkv_paged_decode_attention_multi.
 */
int pkv_paged_decode_attention_multi_k8(void* out, const void* q, const void* k_pool8, const void* v_pool,
                                        const int32_t* block_table, int32_t max_pages, const int32_t* lens, int32_t B,
                                        int32_t n_query, int32_t Hq, int32_t Hkv, int32_t D, int32_t P, int32_t N,
                                        int32_t max_context, float scale, int32_t partition_tokens,
                                        int32_t prefix_tokens, void* workspace, size_t workspace_bytes, void* stream);

/*
 * pkv_paged_decode_attention_window_k8 -- pkv_paged_decode_attention_window
 * over int8-key pages: the last `window` tokens of each sequence through its
 * ring of pages, keys dequantised as code * scale, values fp16; with k_new and
 * v_new the new token is appended into its ring page in the same launch, its
 * key quantised exactly as pkv_kv_append_k8 does. Arguments, workspace and
 * errors as pkv_paged_decode_attention_window, the key pool being the int8
 * pool above (D in {64, 128}).
 */
int pkv_paged_decode_attention_window_k8(void* out, const void* q, const void* k_new, const void* v_new,
                                         void* k_pool8, void* v_pool, const int32_t* ring_table, int32_t ring_pages,
                                         const int32_t* lens, int32_t B, int32_t Hq, int32_t Hkv, int32_t D, int32_t P,
                                         int32_t N, int32_t window, float scale, int32_t partition_tokens,
                                         void* workspace, size_t workspace_bytes, void* stream);

/*
 * pkv_paged_decode_attention_window_multi_k8 --
 * pkv_paged_decode_attention_window_multi over int8-key pages (keys
 * dequantised as code * scale, values fp16). Arguments and errors as there,
 * the key pool being the int8 pool above.
 */
int pkv_paged_decode_attention_window_multi_k8(void* out, const void* q, const void* k_pool8, const void* v_pool,
                                               const int32_t* ring_table, int32_t ring_pages, const int32_t* lens,
                                               int32_t B, int32_t n_query, int32_t Hq, int32_t Hkv, int32_t D,
                                               int32_t P, int32_t N, int32_t window, float scale,
                                               int32_t partition_tokens, void* workspace, size_t workspace_bytes,
                                               void* stream);

/*
 * pkv_probe_stream_read -- measurement aid (not part of decode): read
 * n_tiles 4 KiB tiles of `base` in the order tile_order gives, with the decode
 * kernel's access pattern (16-byte non-temporal loads per lane, two tiles in
 * flight per wave), to measure the streaming-read rate the decode kernels are
 * compared against (pgsm §4.2 makes decode a KV-read-bound step, so this
 * rate, not the spec sheet, is what the kernels can reach).
 *
 *   base       : device buffer of `bytes` bytes, read only.
 *   tile_order : int32 [n_tiles] device, normally a permutation of
 *                [0, bytes / 4096); entries outside that range are clamped
 *                into it.
 *   waves      : waves to spread the tiles over (consecutive runs per wave).
 *   sink       : int32 [1] device; written only on a 1-in-2^32 fold value,
 *                so the loads cannot be dropped.
 * Errors: PKV_ERR_INVALID_ARG (n_tiles < 0, waves <= 0, bytes below
 * n_tiles * 4096, null or misaligned pointers), PKV_ERR_HIP.
 */
int pkv_probe_stream_read(const void* base, size_t bytes, const int32_t* tile_order, int32_t n_tiles,
                          int32_t waves, int32_t* sink, void* stream);

/*
 * pkv_profile_next_partition_kernel -- measurement aid (not part of decode):
 * the next decode call made on this host thread (any pkv_*decode_attention*
 * entry point) launches its partition kernel -- the kernel that reads the
 * cache -- with hipExtLaunchKernel and these two events, which then record
 * that kernel's start and stop on the call's stream; hipEventElapsedTime
 * gives the kernel's own duration, without the merge kernel or the launch
 * gap between them. The hook is consumed by that next call whether or not it
 * launches (a call that returns an error records nothing). Either event may
 * be NULL.
 *
 *   start_event, stop_event: hipEvent_t, created by the caller (with timing),
 *                  owned by the caller; not for use under stream capture.
 * Returns PKV_OK.
 */
int pkv_profile_next_partition_kernel(void* start_event, void* stop_event);

/* ------------------------------------------------------------------------ */
/* Host page allocator (CPU only; no device calls)                           */
/* ------------------------------------------------------------------------ */

/*
 * A pool of N fixed-size pages handed to sequences on demand (dpshk §4.2:
 * allocate in fixed blocks, give pages back as soon as a request ends or
 * fails; shared system-prompt prefixes are stored once). Policy:
 *   - the free list is FIFO: pages leave from the front, in `free_order`
 *     (NULL = 0, 1, ..., N-1), and return to the back;
 *   - reservations are all-or-nothing: on failure nothing changes;
 *   - shared pages are reference counted; a page returns to the free list
 *     when its count reaches zero.
 * Sequence ids are caller-chosen non-negative int32. One allocator may be used
 * from several threads (calls are serialised internally).
 * Every allocator call may also return PKV_ERR_HOST_MEMORY when host memory
 * for its own tables runs out; the allocator's state is then unspecified and
 * it should be destroyed. No C++ exception leaves the library.
 */
typedef struct pkv_allocator pkv_allocator;

/* Create an allocator over num_pages pages of page_size tokens.
 * free_order: NULL or a permutation of [0, num_pages) (host, copied).
 * Errors: PKV_ERR_INVALID_ARG (bad sizes, not a permutation, null out). */
int pkv_alloc_create(int32_t num_pages, int32_t page_size, const int32_t* free_order,
                     pkv_allocator** out);

/* Destroy an allocator (NULL is a no-op). */
void pkv_alloc_destroy(pkv_allocator* alloc);

/* Grow sequence `seq` to hold at least n_tokens tokens (ceil(n_tokens / P)
 * pages), taking new pages from the free list. On success, if bt_row is not
 * NULL, writes the sequence's whole table into bt_row[0 .. max_pages) (-1
 * past the end) and, if n_pages is not NULL, its page count.
 * Errors: PKV_ERR_INVALID_ARG (negative seq/n_tokens, table wider than
 * max_pages), PKV_ERR_OUT_OF_PAGES. On error nothing changes. */
int pkv_alloc_reserve(pkv_allocator* alloc, int32_t seq, int32_t n_tokens, int32_t* bt_row,
                      int32_t max_pages, int32_t* n_pages);

/* Reserve for B sequences at once, all-or-nothing over the whole batch:
 * seqs[i] grows to n_tokens[i] tokens, pages taken in batch order;
 * block_table [B][max_pages] (host) gets every row. Used once per decode step
 * to add a page to the sequences whose next token starts one. Errors as
 * pkv_alloc_reserve, plus PKV_ERR_INVALID_ARG for a sequence listed twice. */
int pkv_alloc_reserve_batch(pkv_allocator* alloc, int32_t B, const int32_t* seqs,
                            const int32_t* n_tokens, int32_t* block_table, int32_t max_pages);

/* Start the (empty) sequence `seq` with n already-allocated pages (their
 * reference counts go up by one), e.g. a shared system-prompt prefix.
 * Errors: PKV_ERR_INVALID_ARG (seq not empty, page not allocated, duplicate). */
int pkv_alloc_share_prefix(pkv_allocator* alloc, int32_t seq, const int32_t* pages, int32_t n);

/* Release all pages of `seq` in table order (reference count - 1; back to the
 * free list at zero). Unknown sequences are a no-op. Call it on completion
 * and on failure of a request alike. */
int pkv_alloc_free(pkv_allocator* alloc, int32_t seq);

/* Pages currently free (-1 if alloc is NULL). */
int32_t pkv_alloc_free_count(const pkv_allocator* alloc);

/* Copy `seq`'s table into bt_row[0 .. max_pages) (-1 padded) and its page
 * count into *n_pages (0 for an unknown sequence). */
int pkv_alloc_table(const pkv_allocator* alloc, int32_t seq, int32_t* bt_row, int32_t max_pages,
                    int32_t* n_pages);

/* Reference count of `page` into *count. */
int pkv_alloc_refcount(const pkv_allocator* alloc, int32_t page, int32_t* count);

/*
 * Prefix cache. A request's prompt KV can be kept after the request ends and
 * shared by later requests with the same prefix (shared prefixes: dpshk §4.2,
 * pgsm §3.2; reuse across requests: pgsm §4.3).
 *
 * pkv_alloc_cache_insert -- keep the pages of the first n_tokens tokens of
 * `seq` under `key` (a caller-chosen identifier of the prompt, e.g. a hash of
 * its tokens). The cache holds one reference on each page, so the pages outlive
 * the sequence. An existing key is only marked as used. Errors:
 * PKV_ERR_INVALID_ARG (n_tokens <= 0, seq holds fewer tokens' pages).
 *
 * pkv_alloc_cache_lookup -- pages (into `pages`, capacity max_pages; NULL to
 * ask the count only) and token count under `key`; marks it as used. A new
 * sequence starts from them with pkv_alloc_share_prefix. Errors:
 * PKV_ERR_NOT_FOUND, PKV_ERR_INVALID_ARG (capacity too small).
 *
 * pkv_alloc_cache_evict -- drop the entry (its references); unknown keys are
 * a no-op. pkv_alloc_cache_entries -- number of entries (-1 for NULL).
 *
 * Eviction: when a reservation (pkv_alloc_reserve*, pkv_alloc_prepare_append)
 * needs more pages than are free, the least recently used entries (by insert
 * or lookup) are dropped one at a time until it fits -- only if dropping all
 * of them would make it fit; otherwise nothing changes (PKV_ERR_OUT_OF_PAGES).
 */
int pkv_alloc_cache_insert(pkv_allocator* alloc, uint64_t key, int32_t seq, int32_t n_tokens);
int pkv_alloc_cache_lookup(pkv_allocator* alloc, uint64_t key, int32_t* pages, int32_t max_pages,
                           int32_t* n_pages, int32_t* n_tokens);
int pkv_alloc_cache_evict(pkv_allocator* alloc, uint64_t key);
int32_t pkv_alloc_cache_entries(const pkv_allocator* alloc);

/*
 * pkv_alloc_prepare_append -- ready a batch for writing token pos[i] of
 * sequence seqs[i] (copy on write of shared pages). Each table grows to hold
 * the token (as pkv_alloc_reserve); if the page the token lands in is shared
 * (count > 1: a shared prefix, or a cached prompt), the sequence gets a
 * private page in its place, the old page's count drops by one, and the pair
 * (copy_src[k], copy_dst[k]) is reported: the caller copies the old page's
 * contents into the new one on the device (pkv_copy_pages) before the write.
 * Batch order decides who copies: once the others have their own copies, the
 * last sharer keeps the page. All or nothing: planned first, committed only if
 * the free list (after evictions) covers it.
 *   seqs, pos : int32 [B] host (distinct sequences, pos >= 0).
 *   copy_src, copy_dst: int32 [B] host, written; *n_copies pairs are used.
 *   block_table: optional int32 [B][max_pages] host: rows of the batch
 *               rewritten (-1 past each table), as pkv_alloc_reserve_batch.
 * Errors: PKV_ERR_INVALID_ARG (duplicates, negatives, a table wider than
 * max_pages), PKV_ERR_OUT_OF_PAGES (nothing changed).
 */
int pkv_alloc_prepare_append(pkv_allocator* alloc, int32_t B, const int32_t* seqs, const int32_t* pos,
                             int32_t* copy_src, int32_t* copy_dst, int32_t* n_copies, int32_t* block_table,
                             int32_t max_pages);

/*
 * pkv_copy_pages -- copy whole pages of one pool on the device: page dst[i]
 * becomes a copy of page src[i] (page_bytes bytes each: Hkv * P * D * 2 for a
 * fp16 pool, pkv_k8_pool_bytes(1, ...) for an int8-key pool). Call it for the
 * K and the V pool with the pairs pkv_alloc_prepare_append reports. The pairs
 * travel in the kernel arguments (64 per launch). src and dst are HOST arrays.
 * Errors: PKV_ERR_INVALID_ARG (a page outside [0, N), a page both copied to
 * and from in one call, page_bytes not a positive multiple of 16, misaligned
 * pool), PKV_ERR_HIP.
 */
int pkv_copy_pages(void* pool, size_t page_bytes, int32_t N, const int32_t* src, const int32_t* dst, int32_t n,
                   void* stream);

/*
 * pkv_validate_tables -- check host copies of a block table and lengths
 * against what the decode entry points assume of device-resident contents.
 * Rules, checked row by row (1-4), then 5, then 6 and 7:
 *   1 lens[b] >= 0;
 *   2 without a window, ceil(lens[b] / P) <= max_pages;
 *   3 every entry a token reaches is in [0, N);
 *   4 no page twice among a row's reached entries;
 *   5 with exclusive_tail != 0, the page of each sequence's last token (where
 *     an append writes) appears in no other row;
 *   6 with prefix_tokens > 0, entries 0 .. prefix_tokens / P - 1 of every
 *     attended row (lens[b] > 0) equal those of the first attended row (the
 *     shared pages of dpshk §4.2, read once for the batch);
 *   7 with prefix_tokens > 0, no attended row is shorter than the prefix.
 * window > 0 reads the table as rings of max_pages pages (the sliding-window
 * entry points): the entries a row reaches are (j % max_pages) for the
 * logical pages j holding tokens max(0, lens[b] - window) .. lens[b] - 1
 * (hotelren §3.2's fixed-capacity buffer), and rule 2 does not apply.
 * Returns PKV_OK or PKV_ERR_INVALID_TABLE with the first offending row and
 * entry in *bad_row / *bad_entry (entry -1 for a length problem) and the rule
 * number in *rule.
 * Errors: PKV_ERR_INVALID_ARG for null pointers, bad sizes, a prefix that is
 * not whole pages, a window with a prefix, or a window that does not fit the
 * ring (window > (max_pages - 1) * P + 1).
 */
int pkv_validate_tables(const int32_t* block_table, const int32_t* lens, int32_t B, int32_t max_pages,
                        int32_t P, int32_t N, int32_t exclusive_tail, int32_t prefix_tokens, int32_t window,
                        int32_t* bad_row, int32_t* bad_entry, int32_t* rule);

#ifdef __cplusplus
}
#endif

#endif /* PKV_H_ */
