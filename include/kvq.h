/*
 * kvq.h — C ABI of the MI355X (gfx950) INT4 KV-cache library.
 *
 * The library implements the serving-side hot path of token-wise INT4
 * KV-cache quantization with a block-diagonal Hadamard rotation:
 *   - kv_quant_append: for every new token, rotate its fp16 K and V per
 *     block, quantize each (token, KV head) vector to INT4 with one fp16
 *     scale, and write the result into a paged cache through a page table,
 *     touching nothing else;
 *   - paged_decode_attn_int4: one decode step of grouped-query attention over
 *     that cache, dequantizing in registers; the query is rotated instead of
 *     the keys, and the output is rotated back;
 *   - paged_decode_step_int4: the two fused for a decode step (each
 *     sequence's new token appended, then attention over its context);
 *   - kv_append_fp16 / paged_decode_attn_fp16: the same two operations on an
 *     unquantized fp16 paged cache, as the baseline.
 *
 * Sources (cited by page title and section):
 *   [EXPL] "KVキャッシュを4ビットへ — SAW-INT4とシステムを踏まえたINT4量子化"
 *          (youngju.dev explainer of the SAW-INT4 preprint):
 *          "KVキャッシュこそが本当のボトルネックである理由" — paged layout and fused
 *          attention as serving constraints;
 *          "素朴なINT4はなぜ崩れるのか" — token-wise INT4, one scale per token,
 *          quantized on arrival and appended, past tokens never revisited;
 *          "回転のトリック — ブロック対角アダマール" — orthogonal, invertible
 *          Hadamard rotation applied within blocks;
 *          "システムこそが設計である — 融合カーネル" and its figure — one fused
 *          kernel: K,V fp16 -> block Hadamard -> token-wise INT4 -> append to
 *          the paged KV block.
 *   [SUMM] "SAW-INT4: System-Aware 4-Bit KV-Cache Quantization for Real-World
 *          LLM Serving" (gist.science summary): the same method, compatible
 *          with paged memory and fused attention.
 *
 * Conventions for every entry point
 *   - Every pointer argument is a DEVICE pointer unless stated otherwise.
 *     The caller allocates and frees every buffer; the library allocates
 *     nothing and keeps no state between calls, and its entry points are
 *     re-entrant, with one exception: paged_decode_attn_int4_noalloc keeps
 *     its partial states in a static per-GPU buffer (see there).
 *   - `stream` is a hipStream_t passed as void* (NULL = the default stream).
 *     Calls only enqueue work on it and return; they never synchronize.
 *   - Return value: KVQ_OK (0) on success, a negative KVQ_ERR_* code
 *     otherwise.  Argument errors are detected on the host before anything is
 *     launched, so a failing call has no effect.  KVQ_ERR_HIP reports a
 *     launch failure from the HIP runtime.
 *   - head_dim must be 128; page_size must be 16 or 32; had_block must be 0
 *     (no rotation: naive INT4), 32, 64 or 128; num_q_heads must be a
 *     multiple of num_kv_heads; pools and workspace must be 16-byte aligned.
 *   - Device-side contract (not checked, because checking would need a
 *     synchronisation): page_table entries that are read lie in
 *     [0, num_pages); (seq, pos) pairs are unique within one append call;
 *     context_lens[b] <= max_context_len <= max_pages_per_seq * page_size.
 *     With the environment variable KVQ_CHECK=1 (read at each call) the
 *     appends, decodes and the prefill copy these indices to the host
 *     (synchronising the stream) and return KVQ_ERR_INVALID_ARG, before any
 *     launch, for a page-table entry outside [0, num_pages), a position past
 *     max_pages_per_seq pages, a context length above max_context_len (the
 *     prefill: above max_pages_per_seq * page_size) or a prefill q_start
 *     that does not run from 0 to num_q without decreasing.  An append's
 *     token_seq entries must name rows the page table has: the calls do not
 *     take its row count, so no mode can check that (KVQ_CHECK copies the
 *     rows up to the largest sequence named).
 *
 * Layouts
 *   K/V input:      fp16 [num_tokens][num_kv_heads][head_dim] (row-major).
 *   Query:          fp16 [batch][num_q_heads][head_dim].
 *   Output:         fp32 [batch][num_q_heads][head_dim].
 *   page_table:     int32 [batch][max_pages_per_seq]: logical page -> physical
 *                   page; position pos of sequence b lives in logical page
 *                   pos / page_size, slot pos % page_size.
 *   INT4 pools:     uint8 [num_pages][num_kv_heads][tile], one pool for K and
 *                   one for V, tile = page_size*head_dim/2 + 2*page_size bytes
 *                   (1056 for P=16, 2112 for P=32), the share of one
 *                   (page, KV head).  One page (num_kv_heads * tile bytes)
 *                   holds first the code rows of KV heads 0..num_kv_heads-1,
 *                   page_size rows of head_dim/2 bytes per head (two's-
 *                   complement nibbles, element 2j in the low nibble of byte
 *                   j), then the scales of heads 0..num_kv_heads-1, page_size
 *                   little-endian fp16 per head:
 *                     code row (h, slot) at  (h * page_size + slot) * head_dim/2
 *                     scale    (h, slot) at  num_kv_heads * page_size * head_dim/2
 *                                            + (h * page_size + slot) * 2
 *                   (every head's codes start on a 1 KiB boundary of the page
 *                   and the scales of 4 heads share one 128-byte line).
 *   fp16 pools:     fp16 [num_pages][num_kv_heads][page_size][head_dim].
 */
#ifndef KVQ_H
#define KVQ_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum {
    KVQ_OK = 0,
    KVQ_ERR_INVALID_ARG = -1,   /* null pointer, negative size, bad combination */
    KVQ_ERR_UNSUPPORTED = -2,   /* head_dim / page_size / had_block outside the supported set */
    KVQ_ERR_WORKSPACE = -3,     /* workspace missing or smaller than required */
    KVQ_ERR_HIP = -4,           /* the HIP runtime reported an error */
    KVQ_ERR_TOO_LARGE = -5      /* the call needs more than the static scratch holds */
};

/* Static, human-readable text for a status code (host function). */
const char *kvq_status_string(int status);

/* Bytes of one (page, KV head) share of an INT4 pool:
 * page_size*head_dim/2 + 2*page_size (a page is num_kv_heads of these; see
 * Layouts).  Returns 0 for unsupported arguments. */
size_t kvq_page_tile_bytes(int32_t head_dim, int32_t page_size);

/*
 * kv_quant_append — fused rotate -> quantize -> paged append ([EXPL] figure
 * in "システムこそが設計である — 融合カーネル"; token-wise scales from
 * "素朴なINT4はなぜ崩れるのか"; block rotation from "回転のトリック").
 *
 * For each token t < num_tokens, each KV head h and each of K, V, with
 * x = the fp16 row k_new[t][h][:] (resp. v_new):
 *   1. y = fp32(x); if had_block > 0, each contiguous block of had_block
 *      entries gets the unnormalised fast Walsh-Hadamard transform in the
 *      fixed order of butterfly spans 1, 2, 4, ... (each butterfly
 *      (u, v) -> (u + v, u - v) is one fp32 operation), then every entry is
 *      multiplied by the fp32 value nearest 1/sqrt(had_block);
 *   2. m = max |y|; scale s = fp16(m / 7) rounded to nearest even;
 *   3. code_i = clamp(round-half-even(y_i / s), -8, 7) with IEEE division
 *      (all codes 0 when s is 0);
 *   4. the D/2 code bytes and s are written to slot token_pos[t] % page_size
 *      of physical page page_table[token_seq[t]][token_pos[t] / page_size].
 * The results are bit-exact with that definition for finite inputs (inf and
 * NaN entries are outside the contract).  No other byte of either pool
 * changes.
 *
 *   k_new, v_new          fp16 [num_tokens][num_kv_heads][head_dim]
 *   token_seq, token_pos  int32 [num_tokens]
 *   page_table            int32 [*][max_pages_per_seq]
 *   k_pool, v_pool        uint8 [num_pages][num_kv_heads][tile], written in place
 * num_tokens == 0 is a no-op returning KVQ_OK.
 */
int kv_quant_append(const uint16_t *k_new, const uint16_t *v_new,
                    const int32_t *token_seq, const int32_t *token_pos, int32_t num_tokens,
                    const int32_t *page_table, int32_t max_pages_per_seq,
                    uint8_t *k_pool, uint8_t *v_pool, int64_t num_pages,
                    int32_t num_kv_heads, int32_t head_dim, int32_t page_size,
                    int32_t had_block, void *stream);

/*
 * Workspace size for the decode entry points: partial softmax states of the
 * split-K reduction (fp32) plus, for batches of 16 to 4096, the prefix sums
 * of the sequences' chunk counts.  The size covers both ways of splitting, so
 * one workspace serves the INT4 and the fp16 decode.  `pages_per_split` = 0
 * lets the library choose (the same choice the decode call makes for the same
 * arguments).
 */
size_t paged_decode_attn_workspace_bytes(int32_t batch, int32_t num_q_heads,
                                         int32_t num_kv_heads, int32_t head_dim,
                                         int32_t max_context_len, int32_t page_size,
                                         int32_t pages_per_split);

/*
 * paged_decode_attn_int4 — one decode step of attention over the INT4 paged
 * cache ([EXPL] "KVキャッシュこそが..." (paged layout, fused attention) and
 * "回転のトリック" (the rotation R = H/sqrt(Bh) is orthogonal and its own
 * inverse, so (R q).(R k) = q.k)).
 *
 * For sequence b, query head qh, KV head h = qh / (num_q_heads/num_kv_heads),
 * L = context_lens[b]:
 *   q' = R q (fp32), keys and values are code * scale read from the tiles,
 *   z_j = softmax_scale * (q' . k_j), w = softmax(z) over j < L,
 *   out[b][qh] = R (sum_j w_j v_j).
 * L <= 0 gives a zero row.  had_block must be the value the cache was
 * written with (0 = no rotation).  Every context_lens[b] must be at most
 * max_context_len (not checked unless KVQ_CHECK=1).  The work is split over
 * page ranges ("split-K"): for batches of 16 to 4096 sequences the chunks
 * (64 tokens) of all sequences are cut into equal ranges, which may run from
 * one sequence into the next; otherwise each sequence is cut into equal
 * ranges of at most 2048 tokens.  Partial softmax states go to `workspace`
 * and a second kernel merges them, so the result does not depend on the
 * split beyond fp32 rounding.  (For tests and measurement, the environment
 * variable KVQ_RANGE_WAVES = 1, 2 or 4, read at each call, sets how many
 * waves of a block share one page range in the per-sequence split schedule
 * of this token-wise INT4 decode; the default chooses by the launch size.)
 *
 *   q              fp16 [batch][num_q_heads][head_dim]
 *   k_pool, v_pool uint8 [num_pages][num_kv_heads][tile]
 *   page_table     int32 [batch][max_pages_per_seq]
 *   context_lens   int32 [batch]
 *   out            fp32 [batch][num_q_heads][head_dim]
 *   workspace      >= paged_decode_attn_workspace_bytes(...) bytes of device memory
 *   pages_per_split  0 = library's choice, else about this many pages per
 *                  range (whole 64-token chunks; per-sequence ranges are
 *                  capped at 2048 tokens, batch-wide ranges at 64 chunks)
 *   phase_event    NULL, or a hipEvent_t (as void*) that this call records on
 *                  `stream` after the split-K partial kernel and before the
 *                  merge kernel, so that a caller can time the two kernels
 *                  apart with events recorded before and after the call
 * A context length above max_context_len is read as max_context_len (the
 * row is then wrong, but no buffer is accessed out of bounds).
 * batch == 0 is a no-op returning KVQ_OK.
 */
int paged_decode_attn_int4(const uint16_t *q, const uint8_t *k_pool, const uint8_t *v_pool,
                           int64_t num_pages, const int32_t *page_table,
                           int32_t max_pages_per_seq, const int32_t *context_lens,
                           int32_t batch, int32_t max_context_len, int32_t num_q_heads,
                           int32_t num_kv_heads, int32_t head_dim, int32_t page_size,
                           int32_t had_block, float softmax_scale, float *out,
                           void *workspace, size_t workspace_bytes,
                           int32_t pages_per_split, void *phase_event, void *stream);

/*
 * paged_decode_step_int4 — one whole decode step: append each sequence's new
 * token to the INT4 cache and attend over the context that ends with it.
 * [EXPL] "システムこそが設計である — 融合カーネル" (the new token's K,V in fp16 go
 * through rotation and token-wise INT4 into the paged block) together with
 * "KVキャッシュこそが..." (every decode step then attends over the whole paged
 * cache).
 *
 * Same result as kv_quant_append of k_new[b], v_new[b] at position
 * L_b - 1 of sequence b (L_b = context_lens[b], for every b with L_b > 0,
 * the same had_block), followed by paged_decode_attn_int4 with the same
 * arguments: the cache bytes written are identical, and so is the output up
 * to fp32 rounding order.  The work is done in two kernels instead of three:
 * the split-K partial kernel reads positions 0 .. L_b - 2 from the cache, and
 * the work range that ends at position L_b - 2 also quantizes the new token,
 * stores it and takes it into its softmax state (a sequence with L_b = 1 is
 * handled by the merge kernel), so no kernel waits for a separate append.
 *
 *   k_new, v_new   fp16 [batch][num_kv_heads][head_dim], 16-byte aligned:
 *                  the K and V rows of each sequence's new token (the rows of
 *                  a sequence with L_b <= 0 are not read)
 *   k_pool, v_pool written at the new tokens' slots only
 *   other arguments, workspace and errors as for paged_decode_attn_int4.
 * Contract (not checked): the slot of a new token lies in no other
 * sequence's context of this call (in the unfused order the other sequence
 * would read the new codes, here the old ones).
 */
int paged_decode_step_int4(const uint16_t *q, const uint16_t *k_new, const uint16_t *v_new,
                           uint8_t *k_pool, uint8_t *v_pool, int64_t num_pages,
                           const int32_t *page_table, int32_t max_pages_per_seq,
                           const int32_t *context_lens, int32_t batch, int32_t max_context_len,
                           int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                           int32_t page_size, int32_t had_block, float softmax_scale, float *out,
                           void *workspace, size_t workspace_bytes, int32_t pages_per_split,
                           void *phase_event, void *stream);

/*
 * paged_prefill_attn_int4 — causal attention of a prompt's queries over the
 * INT4 paged cache, after the prompt's tokens have been appended
 * (kv_quant_append); [EXPL] "KVキャッシュこそが..." (attention over the paged
 * INT4 blocks, in the prefill and decode regimes) and "回転のトリック" (rotate
 * the queries, rotate the outputs back).
 *
 * Query rows q_start[b] .. q_start[b + 1] - 1 belong to sequence b and are its
 * last q_len_b = q_start[b + 1] - q_start[b] positions: row q_start[b] + i is
 * position p = context_lens[b] - q_len_b + i and, for each query head, gets
 *   softmax over k <= p of softmax_scale * (R q).(R k_k), then R (sum w_k R v_k)
 * (the decode's computation at context length p + 1).
 *
 *   q            fp16 [num_q][num_q_heads][head_dim]
 *   q_start      int32 [batch + 1], device: q_start[0] = 0, nondecreasing,
 *                q_start[batch] = num_q, q_len_b <= context_lens[b]; a
 *                sequence with q_len_b > context_lens[b] gets zero rows
 *                and none of its pages is read
 *   out          fp32 [num_q][num_q_heads][head_dim]
 *   softmax_scale  positive and finite (else KVQ_ERR_INVALID_ARG)
 *   other arguments as for paged_decode_attn_int4.
 * No workspace.  num_q == 0 or batch == 0 is a no-op returning KVQ_OK.
 */
int paged_prefill_attn_int4(const uint16_t *q, const int32_t *q_start, int32_t num_q,
                            const uint8_t *k_pool, const uint8_t *v_pool, int64_t num_pages,
                            const int32_t *page_table, int32_t max_pages_per_seq,
                            const int32_t *context_lens, int32_t batch, int32_t num_q_heads,
                            int32_t num_kv_heads, int32_t head_dim, int32_t page_size,
                            int32_t had_block, float softmax_scale, float *out, void *stream);

/*
 * kv_append_fp16 — baseline append: copy each new token's fp16 K/V rows into
 * fp16 pools [num_pages][num_kv_heads][page_size][head_dim] through the page
 * table.  Same arguments and contract as kv_quant_append without had_block.
 */
int kv_append_fp16(const uint16_t *k_new, const uint16_t *v_new,
                   const int32_t *token_seq, const int32_t *token_pos, int32_t num_tokens,
                   const int32_t *page_table, int32_t max_pages_per_seq,
                   uint16_t *k_pool, uint16_t *v_pool, int64_t num_pages,
                   int32_t num_kv_heads, int32_t head_dim, int32_t page_size, void *stream);

/*
 * paged_decode_attn_int4_noalloc — paged_decode_attn_int4 for callers that
 * cannot allocate device memory (code under HIP-graph capture, tight serving
 * loops, harnesses that forbid hipMalloc): the same computation, kernels and
 * result, with the split-K partial states in a static device buffer of
 * KVQ_SCRATCH_BYTES that the library holds on every GPU it runs on until the
 * process ends, instead of a caller's workspace.
 *   - Allocates nothing: no hipMalloc, no hipFree, no allocating library call.
 *   - A call whose partial states need more than KVQ_SCRATCH_BYTES (what
 *     paged_decode_attn_workspace_bytes reports for the schedule the call
 *     takes) returns KVQ_ERR_TOO_LARGE before anything is launched.
 *   - The buffer of a GPU is found on the first call made with that GPU
 *     current (a runtime lookup, no allocation); `stream` must belong to the
 *     current GPU.
 *   - Every call on one GPU uses the same buffer, which keeps the last call's
 *     contents (nothing in it needs to start at zero): calls on one stream
 *     are ordered, but calls that overlap on one GPU (different streams, or
 *     other threads) race and give wrong results.
 * Other arguments, contract and errors as paged_decode_attn_int4.
 */
#define KVQ_SCRATCH_BYTES ((size_t)32 << 20)
int paged_decode_attn_int4_noalloc(const uint16_t *q, const uint8_t *k_pool, const uint8_t *v_pool,
                                   int64_t num_pages, const int32_t *page_table,
                                   int32_t max_pages_per_seq, const int32_t *context_lens,
                                   int32_t batch, int32_t max_context_len, int32_t num_q_heads,
                                   int32_t num_kv_heads, int32_t head_dim, int32_t page_size,
                                   int32_t had_block, float softmax_scale, float *out,
                                   int32_t pages_per_split, void *phase_event, void *stream);

/*
 * paged_decode_attn_fp16 — baseline decode over fp16 pools: the same
 * computation as paged_decode_attn_int4 with unquantized keys and values and
 * no rotation.  Same arguments, split and workspace as paged_decode_attn_int4
 * without had_block.
 */
int paged_decode_attn_fp16(const uint16_t *q, const uint16_t *k_pool, const uint16_t *v_pool,
                           int64_t num_pages, const int32_t *page_table,
                           int32_t max_pages_per_seq, const int32_t *context_lens,
                           int32_t batch, int32_t max_context_len, int32_t num_q_heads,
                           int32_t num_kv_heads, int32_t head_dim, int32_t page_size,
                           float softmax_scale, float *out, void *workspace,
                           size_t workspace_bytes, int32_t pages_per_split,
                           void *phase_event, void *stream);

/*
 * Quantizer variants ("BitDecoding-FP4:FP4 KVキャッシュのネイティブ復号", section
 * 深掘り分析: with one scale per token a single outlier widens the range of
 * the whole token, so smoothing and a Hadamard rotation spread outliers and
 * a scale search picks a scale per group; opening summary: 4-bit
 * microscaling KV formats, NVFP4 / MXFP4; "KVキャッシュを4ビットへ", section
 * 回転のトリック: block-diagonal Hadamard in the QuaRot / SpinQuant line of
 * rotations, whose randomized form multiplies by a random +-1 diagonal).
 *
 * A configuration (a HOST pointer, read during the call):
 *   format        KVQ_FORMAT_INT4: INT4 codes, fp16 scales;
 *                 KVQ_FORMAT_MXFP4: E2M1 codes, one E8M0 scale per 32 channels
 *   had_block     0, 32, 64, 128, as for kv_quant_append
 *   scale_group   channels per scale: INT4 128 (one per token and head: the
 *                 method itself), 64 or 32 (one per Hadamard block when equal
 *                 to had_block); MXFP4 32
 *   scale_search  INT4: 0 = absmax / 7; 1 = search over clipping ratios;
 *                 MXFP4: 0
 *   sign_mask     randomized Hadamard: bit i (word i / 32, bit i % 32) set
 *                 negates channel i before the rotation; all zero = plain
 * Computation, for each vector x (fp16 [128]) and each group of scale_group
 * channels of y = R (S x) (S the sign mask, R the block rotation as in
 * kv_quant_append, fp32 in the same order):
 *   INT4, no search: s = fp16(m / 7) with m the group's absmax, codes as in
 *     kv_quant_append;
 *   INT4, search: among s_k = fp16(fp32(m (16 - k) / 16) / 7), k = 0..7,
 *     the one whose codes give the smallest sum over the group of D^2,
 *     D = round-half-even((y - s_k c) 2^(12 - E)) with m < 2^E (an exact
 *     integer), ties to the smaller k;
 *   MXFP4: scale 2^X with X = floor(log2 m) - 2 (byte X + 127; 0 for an
 *     all-zero group), each element the E2M1 value {0, .5, 1, 1.5, 2, 3, 4,
 *     6} nearest y / 2^X (ties to the code with a zero mantissa bit,
 *     saturating at 6), sign bit set iff y < 0.
 * Layout: a page holds the code rows of every KV head (page_size x 64 bytes
 * each, as for INT4), then the scales: (128 / scale_group) per (head, slot),
 * (head, slot, group) at num_kv_heads * page_size * 64 +
 * ((head * page_size + slot) * (128 / scale_group) + group) * scale_bytes,
 * scale_bytes 2 (fp16, little-endian) or 1 (E8M0).
 */
enum { KVQ_FORMAT_INT4 = 0, KVQ_FORMAT_MXFP4 = 1 };

typedef struct kvq_quant_config {
    int32_t format;
    int32_t had_block;
    int32_t scale_group;
    int32_t scale_search;
    uint32_t sign_mask[4];
} kvq_quant_config;

/* Bytes of one (page, KV head) share of a pool under `cfg`:
 * page_size * 64 + page_size * (128 / scale_group) * scale_bytes; 0 for
 * unsupported arguments. */
size_t kvq_page_tile_bytes_cfg(int32_t head_dim, int32_t page_size, const kvq_quant_config *cfg);

/*
 * kv_quant_append_cfg — kv_quant_append under a quantizer configuration:
 * the same arguments with `cfg` (host pointer) in place of had_block; pools
 * uint8 [num_pages][num_kv_heads][kvq_page_tile_bytes_cfg(...)].  The stored
 * bytes are bit-exact with the definition above.  cfg = {INT4, Bh, 128, 0,
 * 0} is exactly kv_quant_append.
 */
int kv_quant_append_cfg(const uint16_t *k_new, const uint16_t *v_new,
                        const int32_t *token_seq, const int32_t *token_pos, int32_t num_tokens,
                        const int32_t *page_table, int32_t max_pages_per_seq,
                        uint8_t *k_pool, uint8_t *v_pool, int64_t num_pages,
                        int32_t num_kv_heads, int32_t head_dim, int32_t page_size,
                        const kvq_quant_config *cfg, void *stream);

/*
 * paged_decode_attn_cfg — paged_decode_attn_int4 over a cache written by
 * kv_quant_append_cfg with the same `cfg` (host pointer) in place of
 * had_block: q' = R (S q) (S the sign mask, R the block rotation), keys and
 * values dequantized with their group's scale (fp16, or 2^X for MXFP4
 * E2M1 codes), z_j = softmax_scale * (q' . k_j), w = softmax(z),
 * out = S R (sum_j w_j v_j).  Workspace, split, context contract and errors
 * as paged_decode_attn_int4 (paged_decode_attn_workspace_bytes gives the
 * size).  cfg = {INT4, Bh, 128, *, 0} is exactly paged_decode_attn_int4.
 */
int paged_decode_attn_cfg(const uint16_t *q, const uint8_t *k_pool, const uint8_t *v_pool,
                          int64_t num_pages, const int32_t *page_table,
                          int32_t max_pages_per_seq, const int32_t *context_lens,
                          int32_t batch, int32_t max_context_len, int32_t num_q_heads,
                          int32_t num_kv_heads, int32_t head_dim, int32_t page_size,
                          const kvq_quant_config *cfg, float softmax_scale, float *out,
                          void *workspace, size_t workspace_bytes, int32_t pages_per_split,
                          void *phase_event, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* KVQ_H */
