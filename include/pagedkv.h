/*
 * pagedkv.h — C ABI of the MI355X (gfx950) paged decode-attention library.
 *
 * The library implements the decode-time hot path of a block-paged KV cache:
 *   1. kv_cache_append: scatter each new token's K and V rows into a physical
 *      block through a slot mapping;
 *   2. paged_decode_attention: one query per sequence attends over its cached
 *      tokens, gathered page by page through a per-sequence block table,
 *      computing softmax(q K^T * scale) V, optionally restricted to a sliding
 *      window plus sink tokens, or to a per-step list of selected pages.
 *
 * Sources (web pages; cited by title and section):
 *   [primer]  KV-cache primer "从一次线上事故说起：为什么聊到第三十轮，响应突然卡住了" (cf-1.com):
 *             §2.2 (decode appends the new token's K/V, then attends over all cached tokens),
 *             §3.1 (KV-size formula), §4.1 (PagedAttention: fixed 16-token blocks that need
 *             not be contiguous, mapped by a per-sequence block table), §4.3 (sliding window).
 *   [OVAL]    "OVAL — Output-Aware Local Page Bases for KV Cache Retrieval" (2kiu.com):
 *             §2.2 and §3.3 (a small integer array of page base indices chosen per step;
 *             32-token pages stored contiguously), §3.2 (window clamped to [0, cache length),
 *             never reading uninitialised memory past the cache length).
 *   [Novita]  "How KV Sparsity Achieves 1.5x Acceleration for vLLM" (Novita AI blog):
 *             §關鍵技術 1 (per-layer choice of full cache or sliding window over one unified
 *             paged memory), §關鍵技術 2 (one-pass online softmax; the kernel keeps rowmax and
 *             the running sum l, which can be exported at negligible cost).
 *   [naive]   koas-w blog "naive KV cache" post (2026-03-25), §"KV cache的思想": one write
 *             position per step, shared by all layers, advanced once after the last layer.
 *   [TF]      "Transformer模型中的KV Cache优化推理策略" (yutianautomatic.com), §"为什么传统推理方式
 *             难以为继？" (Attention = softmax(Q K^T / sqrt(d_k)) V) and §"增量解码的接口设计"
 *             (the new token attends over cached plus new keys).
 *
 * Conventions for every entry point:
 *   - Pointers are DEVICE pointers unless the comment says "host". The caller owns
 *     every buffer (including workspaces); the library never allocates or frees
 *     device memory (the host block manager's own host memory is allocated by
 *     pkv_bm_create and freed by pkv_bm_destroy) and keeps no state between calls
 *     other than the device error word (pkv_device_errors), the scratch of
 *     paged_decode_attention_noalloc, a thread's profiling events (pkv_profile_events)
 *     and per-device properties it asks the runtime for once (compute units,
 *     occupancy), so calls are reentrant.
 *   - `stream` is a hipStream_t passed as void* (NULL = the null stream). Work is
 *     enqueued asynchronously; no entry point other than pkv_device_errors
 *     synchronises the host.
 *   - The return value reports host-side argument validation and launch errors
 *     only. Validation happens before anything is enqueued: on any error nothing
 *     is launched and no output is touched.
 *   - Device-side preconditions (listed per call) are not checked on the host.
 *     Where a violation could address memory outside the caller's buffers the
 *     kernels skip the offending element instead (documented per call), so a bad
 *     index never faults; the result for that sequence is then unspecified, and a
 *     PKV_DEV_* bit is set in the device error word (pkv_device_errors).
 *
 * Cache layout ("lane-chunk order"). Both pools are arrays of
 *   num_blocks x num_kv_heads page tiles, each tile holding block_size x head_dim
 * elements of the cache dtype; the tile of (block, head) starts at element
 *   (block * num_kv_heads + head) * block_size * head_dim.
 * Within a tile, tokens come in sub-tiles of 16 (block_size is a multiple of 16):
 * token t lives in sub-tile t / 16, which starts at element (t / 16) * 16 * head_dim.
 * A sub-tile is a sequence of 16-byte chunks of E = 16 / sizeof(element) elements
 * (E = 8 for bf16/fp16, 4 for fp32). With tau = t % 16, the element (tau, x),
 * x in [0, head_dim), sits at  chunk * E + pos  where
 *   K:  chunk = (x / (4E)) * 64 + ((x / E) % 4) * 16 + tau,       pos = x % E
 *   V:  R = E / 4, n = x / 16, c = x % 16, j = tau / 4, i = tau % 4,
 *       chunk = ((n / R) * 4 + j) * 16 + c,                      pos = (n % R) * 4 + i
 * Every chunk a wavefront lane feeds to a matrix instruction is then one
 * contiguous 16-byte load, and the 64 lanes of a wavefront read 1 KiB of
 * consecutive bytes per load. The order is a bijection on each sub-tile, so the
 * pool size equals that of a dense [num_blocks][num_kv_heads][block_size][head_dim]
 * array. The order is the library's: only kv_cache_append and the fused decode step
 * (paged_decode_append_attention) write a pool, and only the attention calls read it; a
 * prefill or any other writer goes through kv_cache_append. (The dense order was built and
 * timed too: V then has to be turned on chip, through LDS, into the matrix instruction's
 * operand order, and the Llama-3-8B-shaped decode step took 65.8 us against 60.2 us.)
 */
#ifndef PAGEDKV_H
#define PAGEDKV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    PKV_OK = 0,
    PKV_ERR_NULL = 1,        /* a required pointer is NULL */
    PKV_ERR_SHAPE = 2,       /* a size is non-positive or inconsistent (e.g. Hq % Hkv != 0) */
    PKV_ERR_UNSUPPORTED = 3, /* dtype / head_dim / block_size / group size not built */
    PKV_ERR_MODE = 4,        /* window and page_list both set, or a bad sparsity field */
    PKV_ERR_WORKSPACE = 5,   /* workspace NULL or smaller than the size query returns */
    PKV_ERR_HIP = 6,         /* the HIP runtime reported a launch error */
    PKV_ERR_NO_BLOCKS = 7,   /* block manager: a pool has too few free blocks (nothing changed) */
    PKV_ERR_SCRATCH = 8      /* paged_decode_attention_noalloc: the call needs more workspace than
                                its fixed scratch holds (nothing launched) */
} pkv_status;

typedef enum { PKV_F32 = 0, PKV_F16 = 1, PKV_BF16 = 2, PKV_I8 = 3 } pkv_dtype;

/* Shape of one layer's cache (one K pool and one V pool, same shape and dtype).
 * Supported: dtype in {F32, F16, BF16, I8}; head_dim in {64, 128};
 * block_size a multiple of 16 in [16, 256].
 *
 * INT8 caches ([primer] §4.2 and §5.2: an int8 KV cache dtype halves the bytes per
 * token). A PKV_I8 pool is one buffer: an int8 data plane of num_blocks x num_kv_heads x
 * block_size x head_dim bytes in the lane-chunk order below (E = 16), followed by an fp32
 * scale plane [num_blocks][num_kv_heads][block_size], one scale per (token, kv head) row:
 * element value = int8 * scale. kv_cache_append quantises each appended row
 * symmetrically: amax = max |x| (fp32), scale = amax / 127, q = rint(x * (127 / amax))
 * clamped to [-127, 127], both divisions correctly rounded in fp32 (round to nearest
 * even); a zero row gets scale 0. Rows are never re-quantised. q, k_new and v_new of an
 * INT8 cache are of input_dtype (BF16 or F16). Attention over an INT8 cache always uses
 * the work-split path (split_tokens must be 0, else PKV_ERR_UNSUPPORTED), and the partial
 * call does not accept it (PKV_ERR_UNSUPPORTED). */
typedef struct {
    int32_t num_blocks;   /* physical blocks in each pool */
    int32_t block_size;   /* tokens per block (page size P) */
    int32_t num_kv_heads; /* Hkv */
    int32_t head_dim;     /* d */
    pkv_dtype dtype;      /* element type of the pools, and of k_new/v_new and q unless I8 */
    pkv_dtype input_dtype; /* PKV_I8 only: type of q, k_new, v_new (BF16 or F16) */
} pkv_cache_desc;

/* Which cached tokens one decode step attends to, and a tuning knob.
 * A NULL pointer means full attention with automatic splitting. For a sequence
 * of context length L (the new token included, at position L-1):
 *   full:    tokens [0, L).
 *   window:  window > 0 and window < L: the last `window` tokens [L-window, L)
 *            plus the first min(num_sinks, L) tokens, each token once
 *            ([primer] §4.3; [Novita] §關鍵技術 1). window >= L is full attention.
 *   pages:   page_list != NULL: the tokens of the listed logical pages,
 *            page p covering [p*P, min((p+1)*P, L)) ([OVAL] §2.2, §3.3). The list is
 *            row b of a [batch][pages_per_seq] int32 device array; entries < 0 are
 *            padding. Preconditions: the non-negative entries of a row are
 *            distinct and ascending. Pages starting at or past L contribute nothing
 *            and their block-table entries are never read.
 * window > 0 together with page_list is PKV_ERR_MODE. num_sinks is ignored
 * unless window > 0.
 *
 * Score export ([Novita] §關鍵技術 2: a token's sparsification score is its softmax
 * probability p = exp(q.k - rowmax) / l, summed over recent queries; the attention pass
 * already holds rowmax and l). With score_acc != NULL the call also does, for every
 * sequence b, kv head h and attended token t, with B = max(score_block, 1):
 *     score_acc[b][h][t / B] += sum over the query heads g of kv head h of softmax_g(t),
 * with softmax_g the attention weights of this call: per token for B = 1, per page for
 * B = block_size. Entries without attended tokens are left unchanged, so passing the same
 * array on every step accumulates scores over steps (the caller zeroes or decays it as its
 * policy wants). score_acc is a [batch][num_kv_heads][score_stride] fp32 device array with
 * score_stride >= ceil(min(max_context_len, max_blocks_per_seq * block_size) / B) (else
 * PKV_ERR_SHAPE). Score export runs in the attention kernel of the one-kernel path (the
 * workgroup holding a (sequence, kv head) adds its scores after its own merge) or, on the
 * work-split path, in a kernel after the merge; over a page list with 1 < B != block_size it
 * always takes the work-split path. It needs split_tokens == 0 (else PKV_ERR_MODE) and is not
 * available to paged_decode_attention_partial (PKV_ERR_MODE). Every entry's update is made by
 * one thread, in a fixed order: results do not depend on timing.
 *
 * Ring block tables ([Novita] §關鍵技術 1: a layer may keep a sliding window instead of the
 * full cache, and then needs fewer blocks; [primer] §4.3). With ring_pages = R > 0 (only
 * together with window > 0, else PKV_ERR_MODE) row b of block_table is a ring: with
 * sink_pages = ceil(num_sinks / P), logical page j is read from column j when
 * j < sink_pages and from column sink_pages + (j - sink_pages) mod R otherwise, so the
 * block of page j is reused by page j + R. R must be at least pkv_ring_pages(window, P),
 * the most pages `window` consecutive tokens touch (else PKV_ERR_MODE): then a block is
 * only reused once none of its tokens is attended, and the attended tokens are exactly
 * those of the window mode. max_blocks_per_seq (the row width) must be at least
 * sink_pages + R (else PKV_ERR_SHAPE) and no longer limits the context length. The slots
 * of appended tokens follow the same columns (pkv_bm_append computes them). */
typedef struct {
    int32_t window;          /* <= 0: no window */
    int32_t num_sinks;       /* >= 0 */
    const int32_t* page_list; /* device, nullable */
    int32_t pages_per_seq;   /* row length of page_list; > 0 when page_list != NULL */
    int32_t split_tokens;    /* 0: automatic work split (see paged_decode_attention).
                                Otherwise fixed split-K partitions of this many tokens,
                                rounded up to a multiple of 16 and clamped to [16, 4096]. */
    float* score_acc;        /* nullable: score export, see above (device) */
    int32_t score_stride;    /* row length of score_acc */
    int32_t score_block;     /* tokens per score entry; 0 or 1: one entry per token */
    int32_t ring_pages;      /* 0: plain block table; > 0: ring table of this many pages (above) */
} pkv_decode_opts;

/* kv_cache_append — decode-step cache write ([primer] §2.2; [naive] §"KV cache的思想";
 * [primer] §4.1 for the block addressing).
 * For every i in [0, num_tokens) with slot_mapping[i] >= 0, with
 * blk = slot / block_size and t = slot % block_size:
 *     K pool element (blk, h, t, x) = k_new[i][h][x]   for all h < Hkv, x < d,
 * and likewise V from v_new. The copy is bit-exact (no conversion).
 *   k_cache, v_cache: the pools (lane-chunk order above), written in place.
 *   k_new, v_new:     [num_tokens][num_kv_heads][head_dim], dtype == desc->dtype.
 *   slot_mapping:     [num_tokens] int32; negative = skip that token.
 * num_tokens == 0 is a no-op. Preconditions: the non-negative slots are distinct
 * (two tokens writing one slot race). Slots >= num_blocks * block_size are
 * skipped by the kernel. */
pkv_status kv_cache_append(const pkv_cache_desc* desc /* host */,
                           void* k_cache, void* v_cache,
                           const void* k_new, const void* v_new,
                           const int32_t* slot_mapping, int32_t num_tokens,
                           void* stream);

/* paged_decode_attention — one query per sequence over its paged cache
 * ([TF] §"为什么传统推理方式难以为继？" for the formula; [primer] §4.1 for the block
 * table; [Novita] §關鍵技術 2 for the one-pass online softmax).
 * For each sequence b and query head h (kv head h / (Hq / Hkv), contiguous groups):
 *     s_t = scale * <q[b][h], K_t>   over the attended tokens t (opts above),
 *     out[b][h] = sum_t exp(s_t - m) V_t / sum_t exp(s_t - m),  m = max_t s_t,
 *     lse[b][h] = m + ln(sum_t exp(s_t - m))    (natural log).
 * Token t of sequence b is read from physical block block_table[b][t / P] at
 * position t % P. With no attended token (L == 0): out = 0, lse = -inf.
 *   q:            [batch][num_q_heads][head_dim], dtype == desc->dtype.
 *   block_table:  [batch][max_blocks_per_seq] int32.
 *   context_lens: [batch] int32, device; L_b includes the token appended this step.
 *   max_context_len (host): an upper bound on every L_b; it sizes the launch grid
 *                 so the call never reads device data on the host (graph-capturable).
 *   scale:        <= 0 selects 1 / sqrt(head_dim).
 *   opts (host):  nullable, see pkv_decode_opts.
 *   out:          [batch][num_q_heads][head_dim] of out_dtype (F32 or desc->dtype).
 *   lse_out:      nullable [batch][num_q_heads] fp32.
 *   workspace:    at least paged_decode_attention_workspace_size(...) bytes,
 *                 device memory, 256-byte aligned; contents on entry are ignored.
 * Work split: with split_tokens == 0 the library launches as many wavefronts as the GPU
 * holds at once and gives each an equal, contiguous share of all (sequence, kv head, 16-token
 * unit) work, whatever the spread of context lengths; shares that end inside a sequence
 * leave partials that a second kernel merges by log-sum-exp. Problems of at most 128
 * attended tokens per sequence run as one kernel without a workspace. With split_tokens > 0
 * the split is the fixed partitioning of paged_decode_attention_partial plus the combine.
 * Kernel-side guards: L_b is clamped to min(max_context_len, max_blocks_per_seq * P);
 * tokens whose block id falls outside [0, num_blocks) are skipped. */
pkv_status paged_decode_attention(const pkv_cache_desc* desc /* host */,
                                  const void* k_cache, const void* v_cache,
                                  const void* q,
                                  const int32_t* block_table, int32_t max_blocks_per_seq,
                                  const int32_t* context_lens,
                                  int32_t batch, int32_t num_q_heads,
                                  int32_t max_context_len,
                                  float scale,
                                  const pkv_decode_opts* opts /* host, nullable */,
                                  void* out, pkv_dtype out_dtype,
                                  float* lse_out,
                                  void* workspace, size_t workspace_bytes,
                                  void* stream);

/* paged_decode_append_attention — one decode step of one layer in one pass: the append of
 * the batch's new tokens followed by attention over the updated cache ([primer] §2.2;
 * [naive] §"KV cache的思想": each step writes the new token's K/V, then attends over all).
 * Same result as kv_cache_append(desc, k_cache, v_cache, k_new, v_new, slot_mapping, batch)
 * followed by paged_decode_attention(...) with the same arguments: the same cache contents
 * and the same outputs. On the work-split path of paged_decode_attention both happen in one
 * kernel (plus the combine, which stores the new rows), on the one-kernel path in that kernel
 * (each (sequence, kv head) workgroup stores its row after its own reads); either way the new
 * token enters attention from k_new/v_new directly. On an INT8 cache (work-split path only)
 * the kernel quantises the new row in registers exactly as kv_cache_append does, so the token
 * enters attention as stored, and the combine stores the quantised row and its scales.
 * Partition-path calls (split_tokens > 0 with several partitions) run a separate append first.
 *   k_new, v_new:  [batch][num_kv_heads][head_dim], row b = sequence b's new token.
 *   slot_mapping:  [batch] int32, the slot of position context_lens[b] - 1 of sequence b
 *                  (block_table[b][(L-1)/P] * P + (L-1) % P); < 0 skips the write.
 * Precondition: slot_mapping[b] >= 0 is that slot whenever context_lens[b] > 0 (with a
 * negative slot the new token's values, quantised on an INT8 cache, are still the ones
 * attended), and no other sequence of the call reads that slot (a page that takes a write
 * belongs to one sequence, as after a copy-on-write of shared pages). Other arguments as in
 * paged_decode_attention; the workspace size is the same. */
pkv_status paged_decode_append_attention(const pkv_cache_desc* desc /* host */,
                                         void* k_cache, void* v_cache,
                                         const void* k_new, const void* v_new,
                                         const int32_t* slot_mapping,
                                         const void* q,
                                         const int32_t* block_table, int32_t max_blocks_per_seq,
                                         const int32_t* context_lens,
                                         int32_t batch, int32_t num_q_heads,
                                         int32_t max_context_len,
                                         float scale,
                                         const pkv_decode_opts* opts /* host, nullable */,
                                         void* out, pkv_dtype out_dtype,
                                         float* lse_out,
                                         void* workspace, size_t workspace_bytes,
                                         void* stream);

/* paged_decode_attention_noalloc — paged_decode_attention for callers that cannot allocate
 * device memory: code under HIP graph capture, tight serving loops, harnesses that forbid
 * allocation. Same arguments, results, validation and error codes as paged_decode_attention,
 * without the workspace: the call's workspace is a scratch array inside the library, one per
 * device, held from the first call on that device until the process ends. The call allocates
 * and frees nothing. The scratch holds 32 MiB (33554432 bytes); a call whose
 * paged_decode_attention_workspace_size(...) exceeds that returns PKV_ERR_SCRATCH before
 * anything is enqueued (the Llama-3-8B-shaped layer of 32 sequences up to 4096 tokens needs
 * about 8 MiB, 24 MiB with score export). Every call on a device shares that device's scratch
 * and leaves its contents behind (nothing in it needs to start at zero): calls that overlap in
 * time on one device, on different streams or from different threads, race and give wrong
 * results; calls ordered on one stream are safe. */
pkv_status paged_decode_attention_noalloc(const pkv_cache_desc* desc /* host */,
                                          const void* k_cache, const void* v_cache,
                                          const void* q,
                                          const int32_t* block_table, int32_t max_blocks_per_seq,
                                          const int32_t* context_lens,
                                          int32_t batch, int32_t num_q_heads,
                                          int32_t max_context_len,
                                          float scale,
                                          const pkv_decode_opts* opts /* host, nullable */,
                                          void* out, pkv_dtype out_dtype,
                                          float* lse_out,
                                          void* stream);

/* Bytes of workspace paged_decode_attention needs for these arguments (0 when
 * the call would need none). Returns 0 as well for arguments that the call
 * would reject; pure host function. */
size_t paged_decode_attention_workspace_size(const pkv_cache_desc* desc /* host */,
                                             int32_t batch, int32_t num_q_heads,
                                             int32_t max_context_len,
                                             const pkv_decode_opts* opts /* host, nullable */);

/* Number of split-K partitions per (sequence, head), S >= 1, that the partial call
 * writes for these arguments (the same plan paged_decode_attention uses), or 0 for
 * rejected arguments. Pure host function. */
int32_t paged_decode_attention_num_splits(const pkv_cache_desc* desc /* host */,
                                          int32_t batch, int32_t max_context_len,
                                          const pkv_decode_opts* opts /* host, nullable */);

/* paged_decode_attention_partial — the split-K first phase, exporting per-split
 * softmax statistics ([Novita] §關鍵技術 2: the attention kernel already holds the
 * running max and sum l and can return them). Partitions: the attended tokens are
 * grouped into aligned 16-token units t / 16 — for full and window attention the units
 * that hold attended tokens, ascending; for a page list every 16-token quarter of every
 * list entry in list order, padding included — and partition s of a sequence takes
 * units [s*U, (s+1)*U), U = split size / 16, S = paged_decode_attention_num_splits(...).
 * For partition s of (b, h), over its tokens t:
 *     m_part[b][h][s] = max_t s_t                       (natural-log units),
 *     l_part[b][h][s] = sum_t exp(s_t - m_part),
 *     o_part[b][h][s][:] = sum_t exp(s_t - m_part) V_t  (unnormalised).
 * An empty partition stores m = -inf, l = 0 and leaves its o_part row unwritten.
 * All arguments as in paged_decode_attention, plus
 *   o_part: [batch][num_q_heads][S][head_dim] fp32;  m_part, l_part: [batch][num_q_heads][S] fp32;
 *   num_splits: S as returned by the query (PKV_ERR_SHAPE otherwise).
 * Partial results from several calls over disjoint token sets (for example
 * different devices holding different pages) combine with paged_decode_combine;
 * paged_decode_attention with S > 1 is exactly this call followed by the combine. */
pkv_status paged_decode_attention_partial(const pkv_cache_desc* desc /* host */,
                                          const void* k_cache, const void* v_cache,
                                          const void* q,
                                          const int32_t* block_table, int32_t max_blocks_per_seq,
                                          const int32_t* context_lens,
                                          int32_t batch, int32_t num_q_heads,
                                          int32_t max_context_len,
                                          float scale,
                                          const pkv_decode_opts* opts /* host, nullable */,
                                          float* o_part, float* m_part, float* l_part,
                                          int32_t num_splits,
                                          void* stream);

/* paged_decode_combine — cross-split log-sum-exp reduction ([Novita] §關鍵技術 2:
 * partial softmax results merge through their max and sum). For each (b, h), over
 * the partitions s with l_part > 0:  M = max_s m_s,  w_s = exp(m_s - M),
 *     out[b][h] = sum_s w_s o_s / sum_s w_s l_s,   lse[b][h] = M + ln(sum_s w_s l_s).
 * With no such partition: out = 0, lse = -inf. Layouts as in the partial call;
 * out is [batch][num_q_heads][head_dim] of out_dtype (F32, F16 or BF16, rounded to
 * nearest even); lse_out is nullable. */
pkv_status paged_decode_combine(const float* o_part, const float* m_part, const float* l_part,
                                int32_t batch, int32_t num_q_heads, int32_t num_splits,
                                int32_t head_dim,
                                void* out, pkv_dtype out_dtype, float* lse_out,
                                void* stream);

/* paged_select_pages — the next step's page list from page scores ([OVAL] §3.3: each
 * step keeps the k pages of highest weight and passes their ids to attention; the newest
 * pages, which hold the tokens just appended, are always kept). For sequence b with
 * context length L and n = ceil(L / block_size) pages:
 *   weight(p) = sum over h = 0 .. heads-1, in that order, of scores[b][h][p], in fp32;
 *   the newest min(recent, n) pages [n - recent, n) are always taken; of the older pages
 *   the k - recent of largest weight are taken, equal weights going to the lower id;
 *   page_list[b] = the taken ids ascending, then -1 up to k entries (L == 0: all -1).
 * The result is exactly that of the definition (weights summed in the stated order), so it
 * is deterministic and can be compared bit for bit. The rows are valid page_list rows for
 * paged_decode_attention with pages_per_seq = k.
 *   scores:        [batch][heads][stride] fp32, device: e.g. the score_acc array of a
 *                  decode call with score_block == block_size.
 *   context_lens:  [batch] int32, device.
 *   page_list:     [batch][k] int32, device, written.
 * Limits: 1 <= k <= 64, 0 <= recent <= k, 1 <= heads, 0 <= stride <= 15360, batch <= 65535
 * (else PKV_ERR_SHAPE / PKV_ERR_UNSUPPORTED). Preconditions: n <= stride for every
 * sequence (pages at or past stride are never read: such a sequence is treated as having
 * stride pages), finite scores. */
pkv_status paged_select_pages(const float* scores, int32_t heads, int32_t stride,
                              const int32_t* context_lens, int32_t batch, int32_t block_size,
                              int32_t k, int32_t recent, int32_t* page_list, void* stream);

/* ---- Per-layer memory policy (host) ---------------------------------------------------
 * [Novita] §關鍵技術 1: every layer takes either a full cache or a sliding window over the
 * one paged memory, with its own block-table strategy, and window layers hold fewer blocks.
 * Layers with the same policy form a group: they share one block table and one slot mapping
 * per step (token positions are the same on every layer) and each has its own pools of the
 * group's num_blocks blocks ([naive] §"KV cache的思想": one write position per step serves
 * all layers). A full group gives a sequence one block per page ([primer] §4.1); a window
 * group keeps ceil(S / P) sink blocks plus a ring of R blocks, reused as the window moves.
 * The manager is host code: it hands out block ids and slots; the caller copies tables and
 * slots to the device. It is not thread-safe; calls on one manager must not overlap. */

/* The least ring size for a window of `window` tokens: the most pages that many consecutive
 * tokens touch, floor((window + 2 * block_size - 2) / block_size); 0 when window <= 0 or
 * block_size <= 0. */
int32_t pkv_ring_pages(int32_t window, int32_t block_size);

/* Blocks a sequence of context_len tokens holds in one layer: ceil(L / P) for a full layer
 * (window <= 0); min(ceil(L / P), ceil(S / P) + R) for a window layer, R = ring_pages or,
 * when ring_pages is 0, pkv_ring_pages(window, P). -1 on bad arguments. Times
 * 2 x kv_heads x head_dim x P x element bytes it is the layer's share of the [primer] §3.1
 * KV size. */
int64_t pkv_policy_blocks(int64_t context_len, int32_t block_size, int32_t window, int32_t num_sinks,
                          int32_t ring_pages);

typedef struct pkv_block_manager pkv_block_manager;

typedef struct {
    int32_t window;     /* <= 0: full cache; > 0: sliding window of this many tokens (ring table) */
    int32_t num_sinks;  /* window > 0: the first num_sinks tokens are kept as well (>= 0) */
    int32_t ring_pages; /* window > 0: ring size R; 0 selects pkv_ring_pages(window, block_size) */
    int32_t num_blocks; /* blocks in each pool of the group's layers (ids 0 .. num_blocks - 1) */
} pkv_layer_group;

/* Creates a manager for sequences 0 .. max_seqs - 1 (all empty) over num_groups groups.
 * block_size: a multiple of 16 in [16, 256]. max_pages_per_seq: the row width of a full
 * group's table, so its longest sequence is max_pages_per_seq * block_size tokens.
 * Errors: PKV_ERR_NULL (groups or out NULL), PKV_ERR_SHAPE (non-positive sizes, negative
 * sinks or blocks), PKV_ERR_MODE (ring_pages below the least size), PKV_ERR_UNSUPPORTED
 * (block_size, or num_blocks * block_size beyond int32). *out is set only on success. */
pkv_status pkv_bm_create(int32_t block_size, int32_t max_seqs, int32_t max_pages_per_seq,
                         const pkv_layer_group* groups /* host [num_groups] */, int32_t num_groups,
                         pkv_block_manager** out);
void pkv_bm_destroy(pkv_block_manager* bm);

/* Row width of group g's block table: max_pages_per_seq for a full group, sink pages + R for a
 * window group (the max_blocks_per_seq to pass with it; a window group's row goes with
 * opts.ring_pages = pkv_bm_ring_pages). 0 for a bad group. */
int32_t pkv_bm_table_cols(const pkv_block_manager* bm, int32_t group);
/* R of a window group; 0 for a full group or a bad group. */
int32_t pkv_bm_ring_pages(const pkv_block_manager* bm, int32_t group);

/* Appends num_new[i] tokens to sequence seq_ids[i], i < n (num_new NULL: one token each, a
 * decode step). Blocks are taken from each group's free list as pages are first reached
 * (every page of a full group; every column of a window group's ring, after which blocks are
 * reused). Writes, for group g and the k-th new token in call order (sequence by sequence,
 * positions ascending), slots[g * T + k] = block * block_size + position % block_size, with
 * T = the total of num_new; a window group writes -1 instead for a token that is neither a
 * sink nor among the last `window` tokens once all of the call's tokens are in, so that no
 * two tokens of one call share a slot. context_lens (nullable, [n]) receives the new lengths.
 * All or nothing: PKV_ERR_SHAPE (seq id out of range or repeated, negative count, a full
 * group's row or int32 length exceeded) and PKV_ERR_NO_BLOCKS change nothing. */
pkv_status pkv_bm_append(pkv_block_manager* bm, const int32_t* seq_ids /* host [n] */,
                         const int32_t* num_new /* host [n], nullable */, int32_t n,
                         int32_t* slots /* host [num_groups][T] */,
                         int32_t* context_lens /* host [n], nullable */);

/* Returns every block of sequence seq_id to the free lists and sets its length to 0. */
pkv_status pkv_bm_release(pkv_block_manager* bm, int32_t seq_id);

/* Copies the rows of seq_ids[0 .. n-1] of group g's table into table ([n][cols], host).
 * Columns not yet given a block hold -1 (attention never reads them). */
pkv_status pkv_bm_block_tables(const pkv_block_manager* bm, int32_t group, const int32_t* seq_ids, int32_t n,
                               int32_t* table);

/* Context length of a sequence; -1 for a bad id. */
int64_t pkv_bm_context_len(const pkv_block_manager* bm, int32_t seq_id);
/* Blocks of group g held by all sequences (the sum of pkv_policy_blocks over them); -1 for
 * a bad group. */
int64_t pkv_bm_blocks_in_use(const pkv_block_manager* bm, int32_t group);

/* Profiling hook (measurement only). Sets, for the calling host thread, two hipEvent_t
 * handles (passed as void*) that every later decode call of that thread (paged_decode_attention,
 * _append_attention, _noalloc, _partial) records on its stream right before its main attention
 * kernel and right after it; (NULL, NULL) clears them. This per-thread pair is the one piece of
 * state the library keeps for the caller. The records add queue work to every call, so the hook
 * stays clear outside measurement. Always returns PKV_OK. */
pkv_status pkv_profile_events(void* start_event, void* stop_event);

/* Device error word. The kernels set these bits when they skip work whose device-side
 * precondition does not hold (they never fault on it):
 *   PKV_DEV_BLOCK_ID  a block-table entry of an attended page outside [0, num_blocks);
 *   PKV_DEV_SLOT      an append slot >= num_blocks * block_size (kv_cache_append, fused step);
 *   PKV_DEV_CONTEXT   context_lens[b] above max_context_len or, with a plain table, above
 *                     max_blocks_per_seq * block_size (the kernels clamp it);
 *   PKV_DEV_PAGES     paged_select_pages: a sequence with more pages than the score stride.
 * Page-list order and slot uniqueness are not checked. */
enum { PKV_DEV_BLOCK_ID = 1, PKV_DEV_SLOT = 2, PKV_DEV_CONTEXT = 4, PKV_DEV_PAGES = 8 };

/* Waits for `stream`, then stores the calling device's error word (an OR of PKV_DEV_* bits
 * since it was last cleared; 0 when clean) in *flags (host) and, with clear != 0, zeroes it.
 * Not for use inside graph capture (it synchronises). Work on other streams of the device
 * may set bits between the read and the clear. Errors: PKV_ERR_NULL, PKV_ERR_HIP. */
pkv_status pkv_device_errors(uint32_t* flags /* host */, int32_t clear, void* stream);

/* Measurement helper: the achievable HBM read rate that the attention kernel's rate is
 * compared with ([primer] §7.1: a decode step reads the whole KV cache, so bandwidth bounds
 * it). Launches one kernel in which each of cus * 4 * waves_per_simd wavefronts streams its own
 * contiguous share of buf with 16-byte nontemporal loads (the attention kernel's load form)
 * and discards the bytes; time it with events on `stream`.
 *   buf, bytes:      the buffer to read (device); each wave reads bytes / waves rounded down
 *                    to a multiple of 8 KiB, so *bytes_read (host) <= bytes is what is read.
 *   waves_per_simd:  1..8.
 *   sink:            [sink_len] uint32, sink_len >= cus * 4 * waves_per_simd; written only for
 *                    one value pattern of the data (it keeps the loads from being optimised out).
 * Errors: PKV_ERR_NULL; PKV_ERR_SHAPE (waves_per_simd out of range, under 8 KiB per wave, sink
 * too short); PKV_ERR_HIP. */
pkv_status pkv_read_probe(const void* buf, size_t bytes, int32_t waves_per_simd, uint32_t* sink,
                          size_t sink_len, size_t* bytes_read /* host */, void* stream);

/* KV-cache size in bytes by the formula of [primer] §3.1,
 *   2 x batch x layers x kv_heads x head_dim x seq_len x dtype_bytes,
 * with seq_len rounded up to a multiple of block_size when block_size > 0 (a paged
 * cache allocates whole blocks). Pure host function; 0 on negative inputs. */
uint64_t pkv_kv_cache_bytes(int64_t batch, int64_t layers, int64_t kv_heads,
                            int64_t head_dim, int64_t seq_len, int64_t dtype_bytes,
                            int64_t block_size);

/* Static description of a status code. */
const char* pkv_status_string(pkv_status s);

#ifdef __cplusplus
}
#endif

#endif /* PAGEDKV_H */
