/*
 * duo_attn.h -- C ABI of libduoattn, mixed-head attention over a block-paged, per-head circular KV
 * cache, for AMD Instinct MI355X (gfx950).
 *
 * The problem (four web pages on KV-cache sparsity):
 *   - DuoAttention README, abstract and quick-start: some kv heads ("retrieval heads") attend to every
 *     cached token; the others ("streaming heads") keep and attend only the first sink_size tokens
 *     (attention sinks) and the most recent recent_size tokens. The per-head split, sink_size and
 *     recent_size are exactly the arguments of its enable call.
 *   - vLLM issue "Could you support Attention Sink?", sh1ng's comment: a block-paged cache in which a
 *     streaming head's sink tokens sit in block(s) of their own and the other tokens cycle through a
 *     circular buffer (option 3); its worked tables give the ring index (t - sink) mod ring size.
 *   - vLLM issue "Could you support Attention Sink?", ChuanhongLi's comment: the same head may instead
 *     keep whole blocks, the first one as the sink and the newest ones, dropping a middle block when
 *     a new one starts (the block-granular window below, chosen by a negative recent_size).
 *   - transformers PR "[WIP] Dynamic length in static cache", description: a query only needs the
 *     positions up to its own, not the whole allocated cache; lengths therefore live in a device
 *     array read by the kernels, never on the host, and no launch shape depends on them.
 *
 * Conventions for every call:
 *   - Tensor pointers are DEVICE pointers to row-major, contiguous arrays, 16-byte aligned, owned by
 *     the caller. The library never allocates, frees, synchronizes, or reads device data on the host.
 *   - Calls are asynchronous and ordered on `stream` (a hipStream_t; NULL = the default stream).
 *     Buffers must stay alive until the queued work has finished.
 *   - `head_is_retrieval` is a HOST array of num_kv_heads bytes (1 = retrieval head, 0 = streaming
 *     head). It is read during the call; the caller may free it on return.
 *   - q head hq uses kv head hq / (num_q_heads / num_kv_heads) (contiguous grouping).
 *   - On any error the call returns a non-zero status and launches nothing. A failed kernel launch
 *     returns DUO_ERR_HIP.
 *   - Element types: DUO_F32 (float), DUO_F16 (IEEE half), DUO_BF16 (bfloat16). Every tensor of one
 *     call (q, pools, new tokens, out) has the call's dtype. Outputs are rounded to nearest even.
 *
 * Cache layout (shared by all three calls):
 *   k_pool [num_blocks][block_size][head_dim]   (a K page is token-major)
 *   v_pool [num_blocks][head_dim][block_size]   (a V page is channel-major, so that 8 consecutive
 *                                                tokens of one channel are one 16-byte load)
 *   block_table [batch][num_kv_heads][max_blocks_per_head] int32: physical page of each table column.
 *   Each (sequence b, kv head h) owns the row block_table[b][h]. Slot s of a row is row
 *   s % block_size of page block_table[b][h][s / block_size]. Logical position t is stored at:
 *     retrieval head: slot t                       (needs t < max_blocks_per_head * block_size)
 *     streaming head: slot t                       if t < sink_size (the sink pages)
 *                     slot SB*block_size + (t - sink_size) mod (ring_blocks*block_size) otherwise,
 *                     with SB = ceil(sink_size / block_size) sink pages in front of the ring.
 *   A streaming head uses table columns [0, SB + ring_blocks); a retrieval head uses every column.
 *   Page ids outside [0, num_blocks) are clamped into range by the kernels (wrong results, no fault).
 *   Recent window of a streaming head (every attention call), for the query at position p:
 *     recent_size > 0: positions p - recent_size < j <= p (the recent_size newest, p included);
 *     recent_size < 0: block-granular, the -recent_size newest blocks of block_size positions up to
 *                      p's own, that block counting as one however few of its positions exist:
 *                      (floor(p / block_size) + recent_size + 1) * block_size <= j <= p. Blocks are
 *                      aligned at position 0, so the window holds between
 *                      (-recent_size - 1) * block_size + 1 and -recent_size * block_size positions.
 *     recent_size = 0 is rejected (INVALID_ARG) when a streaming head is present. The window's span
 *     W is recent_size or -recent_size * block_size; the ring must hold the span plus the rows of
 *     one call: ring_blocks * block_size >= W + q_len - 1 (q_len = 1 for decode), else CAPACITY.
 *     The append keeps every ring slot either way; only the attention calls apply the window.
 *   Shared sink pages (vLLM attention-sink issue, sh1ng's option 3: the sink block can serve every
 *   request that starts with the same sink tokens): the rows of several sequences may point a
 *   streaming head's sink columns [0, SB) at the same pages when their first sink_size tokens are
 *   identical. Sink pages hold nothing but positions < sink_size, so every sequence that appends
 *   those positions writes the same bits there; attention reads them through each row. Ring pages
 *   and retrieval rows must stay private to one sequence.
 */
#ifndef DUO_ATTN_H
#define DUO_ATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define DUO_ATTN_ABI_VERSION 15

typedef enum { DUO_F32 = 0, DUO_F16 = 1, DUO_BF16 = 2 } duo_dtype_t;

typedef enum {
  DUO_OK = 0,
  DUO_ERR_INVALID_ARG = 1,   /* null/misaligned pointer, non-positive size, bad mask value, aliasing */
  DUO_ERR_UNSUPPORTED = 2,   /* head_dim not in {64,128,256}, block_size not supported */
  DUO_ERR_CAPACITY = 3,      /* ring or table too small for the requested window / chunk */
  DUO_ERR_WORKSPACE = 4,     /* workspace missing or smaller than the size query says */
  DUO_ERR_HIP = 5            /* a HIP launch failed */
} duo_status_t;

/*
 * kv_append_circular -- write t_new new tokens per sequence into the paged cache.
 *
 * Source: vLLM issue "Could you support Attention Sink?" (the circular-buffer tables and option 3)
 * and transformers PR "[WIP] Dynamic length in static cache" (the cache is updated at the new
 * positions before they are attended).
 *
 *   k_pool, v_pool      device, layout above; written.
 *   block_table         device int32 [batch][num_kv_heads][max_blocks_per_head].
 *   k_new, v_new        device [batch][t_new][num_kv_heads][head_dim] of dtype.
 *   seq_lens_before     device int32 [batch]: tokens already written; token i of sequence b goes to
 *                       position seq_lens_before[b] + i.
 *   seq_lens_after      device int32 [batch] or NULL: receives seq_lens_before[b] + t_new. Must not
 *                       alias seq_lens_before.
 *   head_is_retrieval   host uint8 [num_kv_heads].
 *   block_size          power of two in [1, 256].
 * Semantics: the copy is bit-exact. If several new tokens of one streaming head land on the same
 * ring slot, the newest one is what the slot holds afterwards (older ones are not written). Tokens
 * of a retrieval head at positions >= max_blocks_per_head*block_size are not written.
 * Errors: INVALID_ARG (pointers, sizes, aliasing), UNSUPPORTED (head_dim, dtype, block_size),
 *         CAPACITY (streaming heads present and SB + ring_blocks > max_blocks_per_head or
 *         ring_blocks < 1).
 */
int32_t kv_append_circular(void* k_pool, void* v_pool, const int32_t* block_table,
                           int32_t num_blocks, int32_t block_size, int32_t max_blocks_per_head,
                           const void* k_new, const void* v_new, const int32_t* seq_lens_before,
                           int32_t* seq_lens_after, int32_t batch, int32_t t_new,
                           int32_t num_kv_heads, int32_t head_dim, int32_t dtype,
                           const uint8_t* head_is_retrieval, int32_t sink_size, int32_t recent_size,
                           int32_t ring_blocks, void* stream);

/*
 * duo_attn_decode_workspace_size -- bytes of device workspace duo_attn_decode needs for these static
 * sizes (split_tokens as passed to duo_attn_decode; 0 = the library's choice). The library's split
 * size depends on how many kv heads are retrieval heads; this size covers every retrieval/streaming
 * split of the heads. The caller zero-fills the workspace once after allocating it; every completed
 * decode call leaves it ready for the next. It starts with the merge tickets (one per sequence, kv
 * head and chunk of up to 16 q heads, and one per group of 16 splits where a row has more than 16),
 * at offsets fixed by these sizes, so one workspace serves calls with any split size or mask.
 * Returns 0 for invalid sizes.
 */
size_t duo_attn_decode_workspace_size(int32_t batch, int32_t num_q_heads, int32_t num_kv_heads,
                                      int32_t head_dim, int32_t max_blocks_per_head,
                                      int32_t block_size, int32_t split_tokens);

/*
 * duo_attn_decode -- one new query token per sequence attends over its head's visible positions.
 *
 * Source: DuoAttention README (retrieval heads: all positions; streaming heads: sinks + recent
 * window); transformers PR "[WIP] Dynamic length in static cache" (only positions < seq_len);
 * vLLM PR "[Model] Implement DualChunkAttention for Qwen2 Models", review thread (partial attentions
 * merge through their log-sum-exp; the softmax scale is applied in fp32 to q.k).
 *
 *   q                   device [batch][num_q_heads][head_dim] of dtype.
 *   seq_lens            device int32 [batch]: valid tokens INCLUDING the one being decoded (append
 *                       it first). The query sits at position seq_lens[b] - 1.
 *   softmax_scale       multiplies q.k in fp32 (1/sqrt(head_dim) for standard attention).
 *   out                 device [batch][num_q_heads][head_dim] of dtype.
 *   workspace           device, >= duo_attn_decode_workspace_size(...) bytes, zero-filled once.
 *   split_tokens        keys per split-K work item: 0 = library's choice, else a multiple of 128.
 * Visible positions of the query at p = seq_lens[b] - 1: retrieval head j in [0, p]; streaming head
 * j < sink_size or j in its recent window (see the cache layout; within [0, p]). seq_lens[b] = 0
 * yields a zero output row.
 * Retrieval lengths above max_blocks_per_head*block_size are clamped to it.
 * The q heads of a kv head are taken up to 16 at a time (a larger GQA group in chunks of 16, each
 * reading the kv head's keys and values once).
 * Calls sharing one workspace must not run concurrently. The waves of a work item take its key
 * steps as they become free, so the order in which partial sums are added, and with it the last
 * bits of the output, can differ from call to call (every call is within the stated tolerance).
 * Errors: INVALID_ARG, UNSUPPORTED (head_dim, dtype, block_size not a power of two >= 16),
 *         CAPACITY (streaming heads present and
 *         ring_blocks*block_size < the window's span or SB + ring_blocks > max_blocks_per_head),
 *         WORKSPACE.
 */
int32_t duo_attn_decode(const void* q, const void* k_pool, const void* v_pool,
                        const int32_t* block_table, int32_t num_blocks, int32_t block_size,
                        int32_t max_blocks_per_head, const int32_t* seq_lens, int32_t batch,
                        int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim, int32_t dtype,
                        const uint8_t* head_is_retrieval, int32_t sink_size, int32_t recent_size,
                        int32_t ring_blocks, float softmax_scale, void* out, void* workspace,
                        size_t workspace_bytes, int32_t split_tokens, void* stream);

/*
 * duo_attn_append_decode -- kv_append_circular of one token per sequence and duo_attn_decode of
 * that token's queries, in one launch.
 *
 * Source: transformers PR "[WIP] Dynamic length in static cache", description (the cache is
 * updated at the new position, then the query attends up to it) and DuoAttention README (decode
 * over retrieval and streaming heads); the result is that of the two calls in sequence.
 *
 *   q                   device [batch][num_q_heads][head_dim] of dtype (the new tokens' queries).
 *   k_new, v_new        device [batch][1][num_kv_heads][head_dim] of dtype: token b goes to position
 *                       seq_lens_before[b] of every kv head of sequence b, by the slot rule of
 *                       kv_append_circular (retrieval positions past max_blocks_per_head*block_size
 *                       are not written); bit-exact copies.
 *   k_pool, v_pool      device, layout above; the token's slots are written, the rest read.
 *   seq_lens_before     device int32 [batch]: tokens in the cache before the call. The query of
 *                       sequence b sits at position seq_lens_before[b] and sees the keys of
 *                       duo_attn_decode with seq_lens[b] = seq_lens_before[b] + 1.
 *   seq_lens_after      device int32 [batch] or NULL: receives seq_lens_before[b] + 1. Must not
 *                       alias seq_lens_before.
 *   workspace           as for duo_attn_decode (duo_attn_decode_workspace_size gives its size).
 * Other arguments, outputs, the window and the ring requirements: as for duo_attn_decode.
 * Each work item whose keys hold the new position writes the token before reading any key; no
 * other item reads that slot (a retrieval split reads only its own keys, and the ring slot the
 * token takes held a position older than any window), so the launch needs no ordering between
 * items beyond that.
 * Errors: as for duo_attn_decode; also INVALID_ARG (k_new or v_new null or misaligned,
 *         seq_lens_after misaligned or equal to seq_lens_before).
 */
int32_t duo_attn_append_decode(const void* q, const void* k_new, const void* v_new, void* k_pool,
                               void* v_pool, const int32_t* block_table, int32_t num_blocks,
                               int32_t block_size, int32_t max_blocks_per_head,
                               const int32_t* seq_lens_before, int32_t* seq_lens_after,
                               int32_t batch, int32_t num_q_heads, int32_t num_kv_heads,
                               int32_t head_dim, int32_t dtype, const uint8_t* head_is_retrieval,
                               int32_t sink_size, int32_t recent_size, int32_t ring_blocks,
                               float softmax_scale, void* out, void* workspace,
                               size_t workspace_bytes, int32_t split_tokens, void* stream);

/*
 * duo_attn_decode_noalloc -- duo_attn_decode for callers that cannot allocate device memory (code
 * under HIP graph capture, tight serving loops, harnesses that forbid hipMalloc). It takes no
 * workspace: the library keeps one in a static device array of DUO_NOALLOC_SCRATCH_BYTES, one copy
 * on each GPU it runs on, held until the process ends. The call allocates nothing and frees nothing.
 *
 *   Arguments: those of duo_attn_decode without workspace and workspace_bytes; the same semantics,
 *   kernels and results.
 * Each call clears the merge tickets it uses (a fill kernel on `stream`, ahead of the decode), so
 * the array needs no setup; the first call on a device looks up that device's copy. Calls on one
 * GPU share the array: calls that may overlap on one GPU (other streams, other host threads) race
 * and give wrong results; order them on one stream.
 * Errors: as duo_attn_decode; DUO_ERR_WORKSPACE when the shapes need more than
 * DUO_NOALLOC_SCRATCH_BYTES (duo_attn_decode_workspace_size with the same split_tokens bounds what
 * a call needs); DUO_ERR_HIP when the device's copy cannot be found.
 */
#define DUO_NOALLOC_SCRATCH_BYTES ((size_t)16 << 20)
int32_t duo_attn_decode_noalloc(const void* q, const void* k_pool, const void* v_pool,
                                const int32_t* block_table, int32_t num_blocks, int32_t block_size,
                                int32_t max_blocks_per_head, const int32_t* seq_lens,
                                int32_t batch, int32_t num_q_heads, int32_t num_kv_heads,
                                int32_t head_dim, int32_t dtype, const uint8_t* head_is_retrieval,
                                int32_t sink_size, int32_t recent_size, int32_t ring_blocks,
                                float softmax_scale, void* out, int32_t split_tokens,
                                void* stream);

/*
 * duo_attn_prefill_workspace_size -- bytes of device workspace duo_attn_prefill needs for these
 * sizes and this retrieval/streaming split of the kv heads (head_is_retrieval: host, num_kv_heads
 * bytes). A retrieval head's row tiles split their keys over several workgroups whose partial
 * softmax states meet in the workspace. The caller zero-fills the workspace once after allocating
 * it; every completed prefill call leaves it ready for the next. Returns 0 for invalid sizes.
 */
size_t duo_attn_prefill_workspace_size(int32_t batch, int32_t q_len, int32_t num_q_heads,
                                       int32_t num_kv_heads, int32_t head_dim, int32_t dtype,
                                       const uint8_t* head_is_retrieval);

/*
 * duo_attn_prefill -- q_len query rows per sequence (a prompt chunk already appended to the cache)
 * attend causally over their head's visible positions.
 *
 * Source: as for duo_attn_decode; chunked prefill is the DualChunkAttention PR's recommended mode and
 * the DuoAttention README's prefill-chunk-size trade-off (efficiency section).
 *
 *   q                   device [batch][q_len][num_q_heads][head_dim] of dtype.
 *   seq_lens            device int32 [batch]: valid tokens AFTER the chunk was appended; query row
 *                       i sits at position seq_lens[b] - q_len + i (rows at negative positions
 *                       produce zeros).
 *   out                 device [batch][q_len][num_q_heads][head_dim] of dtype.
 *   workspace           device, >= duo_attn_prefill_workspace_size(...) bytes, zero-filled once
 *                       (may be NULL when no kv head is a retrieval head).
 * Visible set of row i at position p: as for decode. Streaming heads need
 * ring_blocks*block_size >= W + q_len - 1 (W the window's span: recent_size, or -recent_size *
 * block_size for the block-granular window) so that the oldest key of the first row is still in
 * the ring.
 * Calls sharing one workspace must not run concurrently.
 * Errors: INVALID_ARG, UNSUPPORTED (head_dim, dtype, block_size not a power of two >= 16),
 *         CAPACITY, WORKSPACE.
 */
int32_t duo_attn_prefill(const void* q, const void* k_pool, const void* v_pool,
                         const int32_t* block_table, int32_t num_blocks, int32_t block_size,
                         int32_t max_blocks_per_head, const int32_t* seq_lens, int32_t batch,
                         int32_t q_len, int32_t num_q_heads, int32_t num_kv_heads,
                         int32_t head_dim, int32_t dtype, const uint8_t* head_is_retrieval,
                         int32_t sink_size, int32_t recent_size, int32_t ring_blocks,
                         float softmax_scale, void* out, void* workspace, size_t workspace_bytes,
                         void* stream);

/*
 * duo_attn_prefill_varlen_workspace_size -- bytes of device workspace duo_attn_prefill_varlen needs
 * for these sizes (total_q and max_q_len as passed to the call; max_blocks_per_head and block_size
 * of the cache) and this retrieval/streaming split (head_is_retrieval: host, num_kv_heads bytes).
 * It covers the prefill row tiles and the split-K decode items of single-row sequences. Zero-fill it once after allocating; every completed call leaves it
 * ready for the next. Returns 0 for invalid sizes.
 */
size_t duo_attn_prefill_varlen_workspace_size(int32_t batch, int32_t total_q, int32_t max_q_len,
                                              int32_t num_q_heads, int32_t num_kv_heads,
                                              int32_t head_dim, int32_t dtype,
                                              int32_t max_blocks_per_head, int32_t block_size,
                                              const uint8_t* head_is_retrieval);

/*
 * duo_attn_prefill_varlen -- duo_attn_prefill for a packed batch in which every sequence brings its
 * own number of query rows (prompt chunks and single decode tokens side by side, as a continuous-
 * batching step does), in one launch.
 *
 * Source: as for duo_attn_prefill; the DualChunkAttention PR's description adds the per-sequence
 * prefill lengths to the attention metadata of a batched step, which is what q_start carries here.
 *
 *   q, out              device [total_q][num_q_heads][head_dim] of dtype: the rows of all sequences,
 *                       packed.
 *   q_start             device int32 [batch + 1]: sequence b owns rows [q_start[b], q_start[b+1]),
 *                       with q_start[0] = 0, non-decreasing, at most max_q_len rows per sequence and
 *                       q_start[batch] <= total_q. The kernels clamp every range into [0, total_q)
 *                       and to max_q_len rows, so malformed offsets give wrong rows, never a fault.
 *   seq_lens            device int32 [batch]: valid tokens AFTER the rows were appended; row i of
 *                       sequence b sits at position seq_lens[b] - n_b + i (n_b its number of rows).
 *   max_q_len           host bound on any sequence's rows: with total_q it sizes the launch (no host
 *                       read of the offsets) and it sets the ring check.
 *   workspace           >= duo_attn_prefill_varlen_workspace_size(...) bytes, zero-filled once.
 * The kernel numbers the row tiles the sequences actually have on the device (from q_start), so the
 * launch holds about total_q / 256 + batch row tiles per head whatever the mix. A sequence with
 * exactly one row (a decode step) is attended by split-K decode items in the same launch, as
 * duo_attn_decode would.
 * Everything else is as for duo_attn_prefill. Errors: as duo_attn_prefill, and INVALID_ARG for a
 * missing or misaligned q_start or total_q, max_q_len < 1.
 */
int32_t duo_attn_prefill_varlen(const void* q, const void* k_pool, const void* v_pool,
                                const int32_t* block_table, int32_t num_blocks, int32_t block_size,
                                int32_t max_blocks_per_head, const int32_t* seq_lens,
                                const int32_t* q_start, int32_t batch, int32_t total_q,
                                int32_t max_q_len, int32_t num_q_heads, int32_t num_kv_heads,
                                int32_t head_dim, int32_t dtype, const uint8_t* head_is_retrieval,
                                int32_t sink_size, int32_t recent_size, int32_t ring_blocks,
                                float softmax_scale, void* out, void* workspace,
                                size_t workspace_bytes, void* stream);

/*
 * The int8 cache -- the same paged, per-head circular layout with 8-bit codes and one fp32 scale per
 * slot for K and one for V.
 *
 * Source: DuoAttention README, installation and usage (the QServe install step and the demo): the
 * retrieval/streaming split is paired with a quantized KV cache, which is how one GPU holds
 * multi-million-token contexts. The pages fix no quantization scheme; this library's is:
 *   amax  = max |x| over one stored row (the head_dim values of one token of one kv head, K and V
 *           separately), exact in fp32;
 *   scale = amax / 127 and inv = 127 / amax, correctly rounded fp32 divisions;
 *   code  = x * inv (correctly rounded fp32 product), rounded half to even, clamped to [-127, 127];
 *   an all-zero row stores codes 0 and scale 0. The row's value is code * scale.
 * Layout:
 *   k_pool  int8 [num_blocks][block_size][head_dim]     (token-major, as the K pages above)
 *   v_pool  int8 [num_blocks][head_dim][block_size]     (channel-major, as the V pages above)
 *   k_scale, v_scale  float [num_blocks][block_size]: the scale of slot row r of page P at [P][r].
 * Block table, slots, lengths and every other convention are those of the calls above. New rows
 * (k_new, v_new) and q / out are DUO_F32, DUO_F16 or DUO_BF16 (the call's dtype). The new rows must
 * be finite.
 */

/*
 * kv_append_circular_int8 -- as kv_append_circular, quantizing each new K and V row: its codes go
 * to the row's slot in the pages and its scale to [page][row] of k_scale / v_scale. Codes and scales
 * are bit-exact functions of the row (the scheme above). Errors: as kv_append_circular, and
 * INVALID_ARG for a missing, misaligned or shared scale pool.
 */
int32_t kv_append_circular_int8(int8_t* k_pool, int8_t* v_pool, float* k_scale, float* v_scale,
                                const int32_t* block_table, int32_t num_blocks, int32_t block_size,
                                int32_t max_blocks_per_head, const void* k_new, const void* v_new,
                                const int32_t* seq_lens_before, int32_t* seq_lens_after,
                                int32_t batch, int32_t t_new, int32_t num_kv_heads,
                                int32_t head_dim, int32_t dtype, const uint8_t* head_is_retrieval,
                                int32_t sink_size, int32_t recent_size, int32_t ring_blocks,
                                void* stream);

/*
 * duo_attn_decode_int8 -- as duo_attn_decode over the int8 cache: a score is softmax_scale times q
 * dotted with the key's codes times the key's K scale, and a value row is its codes times its V
 * scale. The workspace is the one duo_attn_decode_workspace_size gives for the same sizes. Errors:
 * as duo_attn_decode, and INVALID_ARG for a missing or misaligned scale pool.
 */
int32_t duo_attn_decode_int8(const void* q, const int8_t* k_pool, const int8_t* v_pool,
                             const float* k_scale, const float* v_scale,
                             const int32_t* block_table, int32_t num_blocks, int32_t block_size,
                             int32_t max_blocks_per_head, const int32_t* seq_lens, int32_t batch,
                             int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                             int32_t dtype, const uint8_t* head_is_retrieval, int32_t sink_size,
                             int32_t recent_size, int32_t ring_blocks, float softmax_scale,
                             void* out, void* workspace, size_t workspace_bytes,
                             int32_t split_tokens, void* stream);

/*
 * duo_attn_append_decode_int8 -- kv_append_circular_int8 of one token per sequence and
 * duo_attn_decode_int8 of that token's queries, in one launch (see duo_attn_append_decode). The
 * work item that writes the token quantizes it exactly as kv_append_circular_int8 does (the same
 * codes and scale bits). Arguments: those of duo_attn_append_decode, with the int8 pools and
 * their scale pools (written at the token's slot). Errors: as duo_attn_append_decode and
 * duo_attn_decode_int8.
 */
int32_t duo_attn_append_decode_int8(const void* q, const void* k_new, const void* v_new,
                                    int8_t* k_pool, int8_t* v_pool, float* k_scale, float* v_scale,
                                    const int32_t* block_table, int32_t num_blocks,
                                    int32_t block_size, int32_t max_blocks_per_head,
                                    const int32_t* seq_lens_before, int32_t* seq_lens_after,
                                    int32_t batch, int32_t num_q_heads, int32_t num_kv_heads,
                                    int32_t head_dim, int32_t dtype,
                                    const uint8_t* head_is_retrieval, int32_t sink_size,
                                    int32_t recent_size, int32_t ring_blocks, float softmax_scale,
                                    void* out, void* workspace, size_t workspace_bytes,
                                    int32_t split_tokens, void* stream);

/*
 * The 4-bit cache -- the same paged, per-head circular layout with 4-bit codes and one fp32 scale
 * per kv head and channel for K and one for V.
 *
 * Source: DuoAttention README, installation section (the "w8a8kv4-per-channel" demo models) and
 * efficiency section (8-bit weights and a 4-bit KV cache hold 3.3 million tokens of Llama-3-8B on
 * one A100-80G). The pages fix no scheme beyond "4-bit" and "per channel"; this library's is:
 *   scales   k_scale, v_scale float [num_kv_heads][head_dim], set by the caller (calibrated
 *            offline) and the same for every token, so a new row is quantized on its own;
 *   code     = x / s (a correctly rounded fp32 division) rounded half to even, clamped to [-7, 7];
 *            a channel whose scale is 0 stores code 0. The row's value is code * s.
 *   storage  a code c is the 4-bit number u = c + 8. Eight consecutive codes e0..e7 of a row form a
 *            little-endian 32-bit word: bits 4i..4i+3 hold u(e_2i), bits 16+4i..16+4i+3 hold
 *            u(e_2i+1), i = 0..3.
 * Layout:
 *   k_pool  uint8 [num_blocks][block_size][head_dim / 2]  (token-major: a row is head_dim / 8 words
 *                                                          over channels 0, 1, ...)
 *   v_pool  uint8 [num_blocks][head_dim][block_size / 2]  (channel-major: a row is block_size / 8
 *                                                          words over slots 0, 1, ...)
 * Block table, slots, lengths and every other convention are those of the 16-bit calls. q / out and
 * the new rows are DUO_F16 or DUO_BF16; block_size is at least 16. The new rows must be finite and
 * the scales finite and non-negative.
 */

/*
 * kv_append_circular_int4 -- as kv_append_circular, quantizing each new K and V row with its kv
 * head's scales (the scheme above) into the 4-bit pages. Codes are bit-exact functions of the row
 * and the scales; the other codes of a word (other tokens of a V page row) are left as they were.
 * Errors: as kv_append_circular, INVALID_ARG for a missing or misaligned scale array, UNSUPPORTED
 * for DUO_F32 or block_size < 16.
 */
int32_t kv_append_circular_int4(uint8_t* k_pool, uint8_t* v_pool, const float* k_scale,
                                const float* v_scale, const int32_t* block_table,
                                int32_t num_blocks, int32_t block_size,
                                int32_t max_blocks_per_head, const void* k_new, const void* v_new,
                                const int32_t* seq_lens_before, int32_t* seq_lens_after,
                                int32_t batch, int32_t t_new, int32_t num_kv_heads,
                                int32_t head_dim, int32_t dtype, const uint8_t* head_is_retrieval,
                                int32_t sink_size, int32_t recent_size, int32_t ring_blocks,
                                void* stream);

/*
 * duo_attn_decode_int4 -- as duo_attn_decode over the 4-bit cache: a score is softmax_scale times
 * the sum over channels of q * k_scale * code, and a value row is code * v_scale per channel. The
 * workspace is the one duo_attn_decode_workspace_size gives for the same sizes. Errors: as
 * duo_attn_decode, INVALID_ARG for a missing or misaligned scale array, UNSUPPORTED for DUO_F32.
 */
int32_t duo_attn_decode_int4(const void* q, const uint8_t* k_pool, const uint8_t* v_pool,
                             const float* k_scale, const float* v_scale,
                             const int32_t* block_table, int32_t num_blocks, int32_t block_size,
                             int32_t max_blocks_per_head, const int32_t* seq_lens, int32_t batch,
                             int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                             int32_t dtype, const uint8_t* head_is_retrieval, int32_t sink_size,
                             int32_t recent_size, int32_t ring_blocks, float softmax_scale,
                             void* out, void* workspace, size_t workspace_bytes,
                             int32_t split_tokens, void* stream);

/*
 * duo_attn_append_decode_int4 -- kv_append_circular_int4 of one token per sequence and
 * duo_attn_decode_int4 of that token's queries, in one launch (see duo_attn_append_decode). The
 * work item that writes the token quantizes it exactly as kv_append_circular_int4 does (the same
 * code bits): the K row's words whole, and for V each channel's 4-bit field of the token's slot
 * merged into its word (no other item of the launch changes that word's other fields). Arguments:
 * those of duo_attn_append_decode, with the 4-bit pools and the per-(kv head, channel) scales.
 * Errors: as duo_attn_append_decode and duo_attn_decode_int4.
 */
int32_t duo_attn_append_decode_int4(const void* q, const void* k_new, const void* v_new,
                                    uint8_t* k_pool, uint8_t* v_pool, const float* k_scale,
                                    const float* v_scale, const int32_t* block_table,
                                    int32_t num_blocks, int32_t block_size,
                                    int32_t max_blocks_per_head, const int32_t* seq_lens_before,
                                    int32_t* seq_lens_after, int32_t batch, int32_t num_q_heads,
                                    int32_t num_kv_heads, int32_t head_dim, int32_t dtype,
                                    const uint8_t* head_is_retrieval, int32_t sink_size,
                                    int32_t recent_size, int32_t ring_blocks, float softmax_scale,
                                    void* out, void* workspace, size_t workspace_bytes,
                                    int32_t split_tokens, void* stream);

/*
 * Dual Chunk Attention -- the prefill and decode of the vLLM PR "[Model] Implement DualChunkAttention
 * for Qwen2 Models" over this library's paged cache, each in one launch (the PR's brute-force form
 * calls an attention kernel three times per chunk and merges the results).
 *
 * Source: that PR's description (the rotary layer hands attention three query vectors per token:
 * intra-, succ- and inter-chunk) and review thread (the brute-force prefill swaps q for q_succ or
 * q_inter by the chunk relation of query and key; every chunk but the query's own is chunk_len long;
 * the weight is (q . k) * softmax_scale * mscale with an fp32 mscale per query position, applied in
 * fp32; the partial results are merged by their log-sum-exp, i.e. one softmax over all keys j <= p).
 * With chunk(t) = t / chunk_len, the query at position p uses against key j <= p:
 *   q        if chunk(j) == chunk(p);
 *   q_succ   if chunk(j) == chunk(p) - 1;
 *   q_inter  if chunk(j) <  chunk(p) - 1.
 * Every kv head is a full causal head (no streaming heads), bounded by the sequence's valid length,
 * so the cache is filled with kv_append_circular with every kv head marked retrieval.
 */

/*
 * dca_attn_prefill_workspace_size -- bytes of device workspace dca_attn_prefill needs (the
 * duo_attn_prefill workspace with every kv head a retrieval head); zero-fill it once after
 * allocation. Returns 0 for invalid sizes.
 */
size_t dca_attn_prefill_workspace_size(int32_t batch, int32_t q_len, int32_t num_q_heads,
                                       int32_t num_kv_heads, int32_t head_dim, int32_t dtype);

/*
 * dca_attn_prefill -- q_len query rows per sequence (appended to the cache already) attend over
 * positions 0..p of their kv head with the query vector the chunk relation selects.
 *
 *   q, q_succ, q_inter  device [batch][q_len][num_q_heads][head_dim] of dtype (16-byte aligned):
 *                       the intra-, succ- and inter-chunk query vectors of each row.
 *   mscale              device float [batch][q_len]: the row's factor on softmax_scale; it must be
 *                       positive and finite (other values give wrong rows, never a fault).
 *   chunk_len           chunk length in tokens, a multiple of 64 (so a 64-key tile lies in one chunk).
 *   seq_lens, out, workspace, the pool, table and stream arguments: as for duo_attn_prefill (row i
 *                       at position seq_lens[b] - q_len + i).
 * Supported: dtype DUO_F16 or DUO_BF16, head_dim 64 or 128.
 * Errors: INVALID_ARG (a missing or misaligned pointer, chunk_len < 1, sizes as duo_attn_prefill),
 *         UNSUPPORTED (chunk_len not a multiple of 64, dtype, head_dim, block_size), WORKSPACE.
 */
int32_t dca_attn_prefill(const void* q, const void* q_succ, const void* q_inter,
                         const float* mscale, int32_t chunk_len, const void* k_pool,
                         const void* v_pool, const int32_t* block_table, int32_t num_blocks,
                         int32_t block_size, int32_t max_blocks_per_head, const int32_t* seq_lens,
                         int32_t batch, int32_t q_len, int32_t num_q_heads, int32_t num_kv_heads,
                         int32_t head_dim, int32_t dtype, float softmax_scale, void* out,
                         void* workspace, size_t workspace_bytes, void* stream);

/*
 * dca_attn_decode -- Dual Chunk Attention for one query per sequence (the PR's paged decode beside
 * its prefill): the query at position seq_lens[b] - 1 attends over positions 0..seq_lens[b]-1 of its
 * kv head, choosing q, q_succ or q_inter for each key as above.
 *
 *   q, q_succ, q_inter, out  device [batch][num_q_heads][head_dim] of dtype (16-byte aligned).
 *   mscale              device float [batch]: the sequence's factor on softmax_scale (positive,
 *                       finite).
 *   chunk_len, pools, table, seq_lens: as for dca_attn_prefill.
 *   workspace, split_tokens: as for duo_attn_decode (duo_attn_decode_workspace_size for the same
 *                       sizes and split_tokens).
 * Supported: dtype DUO_F16 or DUO_BF16, head_dim 64 or 128.
 * Errors: as dca_attn_prefill and duo_attn_decode.
 */
int32_t dca_attn_decode(const void* q, const void* q_succ, const void* q_inter,
                        const float* mscale, int32_t chunk_len, const void* k_pool,
                        const void* v_pool, const int32_t* block_table, int32_t num_blocks,
                        int32_t block_size, int32_t max_blocks_per_head, const int32_t* seq_lens,
                        int32_t batch, int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                        int32_t dtype, float softmax_scale, void* out, void* workspace,
                        size_t workspace_bytes, int32_t split_tokens, void* stream);

/*
 * duo_profile_next_launch -- a profiling hook for the caller's own timing. The next attention call
 * (duo_attn_decode, duo_attn_decode_noalloc, duo_attn_decode_int8, duo_attn_decode_int4,
 * duo_attn_prefill, duo_attn_prefill_varlen, dca_attn_prefill, dca_attn_decode) made from this host thread launches its kernel with
 * start_event and stop_event attached to the dispatch itself: the events take the kernel's own
 * start and end times, without the queue's gap before the dispatch. The events (hipEvent_t, timing
 * enabled) are created and owned by the caller; either may be NULL. The hook applies to that one
 * call, which takes it even when it returns an error, and then clears. Always returns DUO_OK.
 */
int32_t duo_profile_next_launch(void* start_event, void* stop_event);

/* Human-readable name of a status code (static storage). */
const char* duo_status_string(int32_t status);

/* DUO_ATTN_ABI_VERSION of the loaded library. */
int32_t duo_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* DUO_ATTN_H */
