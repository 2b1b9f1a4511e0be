/*
 * oracle.c — plain, slow CPU reference for paged decode attention.
 *
 * TEST INFRASTRUCTURE. Only the tests, the smoke check and the benchmark's
 * CPU-baseline leg may load this library; the product path never does. It shares
 * no code, header, table or helper with the HIP library: everything it needs,
 * including the cache layout, is written out again here from its definition.
 *
 * Arithmetic: every input element (fp32, fp16 or bf16) is decoded exactly into a
 * double; dot products, the softmax and the weighted sums run in double in
 * ascending index order; the brute-force path runs in long double.
 *
 * Sources (web pages, by title and section):
 *   [primer] KV-cache primer "从一次线上事故说起：为什么聊到第三十轮，响应突然卡住了"
 *            (cf-1.com): §2.2 decode = append the new token's K/V, then attend over all
 *            cached tokens; §3.1 KV-size formula; §4.1 block table; §4.3 sliding window.
 *   [OVAL]   "OVAL — Output-Aware Local Page Bases for KV Cache Retrieval" (2kiu.com):
 *            §2.2/§3.3 per-step page base indices, the top-k pages by weight; §3.2 window
 *            clamps.
 *   [Novita] "How KV Sparsity Achieves 1.5x Acceleration for vLLM": §關鍵技術 1 per-layer
 *            full cache or sliding window; §關鍵技術 2 online softmax keeping rowmax and l,
 *            and the per-token sparsification score built from them.
 *   [TF]     "Transformer模型中的KV Cache优化推理策略": §"为什么传统推理方式难以为继？"
 *            Attention(Q,K,V) = softmax(Q K^T / sqrt(d_k)) V.
 *
 * Readings where the pages are silent (each listed in the design notes):
 *   - the scale defaults to 1/sqrt(head_dim) ([TF] formula) and may be overridden;
 *   - query head h uses kv head h / (Hq / Hkv) (contiguous GQA groups);
 *   - the window is the last W tokens including the new one, plus the first S
 *     "sink" tokens, each token once; W >= L is full attention;
 *   - page_list entries are logical page ids per sequence, shared by all heads,
 *     translated through the block table; entries < 0 are padding;
 *   - L == 0 gives out = 0 and lse = -inf;
 *   - a token's score sums the softmax probabilities of the query heads that share its
 *     kv head (the cache is per kv head), one query per head per decode step.
 *   - INT8 rows are quantised symmetrically, one fp32 scale per (token, kv head) row;
 *   - a window layer's block table is a ring of ceil(S/P) sink columns plus R columns, R the
 *     most pages W consecutive tokens touch, so a block is reused only when none of its
 *     tokens is attended.
 *
 * Parity status: every function here is pinned by the CPU tests (closed forms,
 * invariants, brute force, the primer's worked KV-size values); none is unpinned.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* ORC_I8_BF16 / ORC_I8_F16: an INT8 cache ([primer] §4.2 and §5.2's int8 KV cache dtype,
 * which halves the bytes per token) whose inputs (q, new K/V rows) are bf16 / fp16. Such a
 * pool holds an int8 data plane [num_blocks][Hkv][P][d] in the same lane-chunk order as
 * the other dtypes (16 elements per 16-byte chunk), followed by an fp32 scale plane
 * [num_blocks][Hkv][P]: one scale per (token, kv head) row. Element value = int8 * scale. */
enum { ORC_F32 = 0, ORC_F16 = 1, ORC_BF16 = 2, ORC_I8_BF16 = 3, ORC_I8_F16 = 4 };
enum { ORC_OK = 0, ORC_ERR_ARG = 1, ORC_ERR_PRECONDITION = 2, ORC_ERR_NOMEM = 3 };

static int is_q8(int dt) { return dt == ORC_I8_BF16 || dt == ORC_I8_F16; }
/* dtype of q and of the rows handed to append */
static int in_dt(int dt) { return dt == ORC_I8_BF16 ? ORC_BF16 : dt == ORC_I8_F16 ? ORC_F16 : dt; }
/* bytes of one cache element */
static size_t elem_size(int dt) { return dt == ORC_F32 ? 4u : is_q8(dt) ? 1u : 2u; }

/* IEEE-754 binary16: 1 sign, 5 exponent (bias 15), 10 fraction bits. */
static double decode_f16(uint16_t h) {
    int sign = (h >> 15) & 1;
    int e = (h >> 10) & 0x1f;
    int f = h & 0x3ff;
    double v;
    if (e == 0)
        v = ldexp((double)f, -24); /* subnormal: f * 2^-14 * 2^-10 */
    else if (e == 31)
        v = f ? NAN : INFINITY;
    else
        v = ldexp((double)(f | 0x400), e - 25); /* (1.f) * 2^(e-15), as an integer * 2^-10 */
    return sign ? -v : v;
}

/* bfloat16: the upper 16 bits of an IEEE binary32. */
static double decode_bf16(uint16_t h) {
    uint32_t u = (uint32_t)h << 16;
    float f;
    memcpy(&f, &u, 4);
    return (double)f;
}

static double load_elem(const void* base, size_t idx, int dt) {
    if (dt == ORC_F32) {
        float f;
        memcpy(&f, (const char*)base + idx * 4, 4);
        return (double)f;
    }
    uint16_t h;
    memcpy(&h, (const char*)base + idx * 2, 2);
    return dt == ORC_F16 ? decode_f16(h) : decode_bf16(h);
}

/* Cache layout, as the library's interface documents it ("lane-chunk order").
 * Element (block blk, kv head h, token-in-block t, dim x) of a pool lives at the
 * returned element index. E = elements per 16-byte chunk. */
static size_t k_index(size_t blk, int h, int t, int x, int Hkv, int P, int d, int dt) {
    int E = (int)(16 / elem_size(dt));
    size_t tile = ((size_t)blk * Hkv + h) * (size_t)P * d;
    size_t sub = (size_t)(t / 16) * 16 * d;
    int tau = t % 16;
    size_t chunk = (size_t)(x / (4 * E)) * 64 + (size_t)((x / E) % 4) * 16 + tau;
    return tile + sub + chunk * E + (size_t)(x % E);
}

static size_t v_index(size_t blk, int h, int t, int x, int Hkv, int P, int d, int dt) {
    int E = (int)(16 / elem_size(dt));
    int R = E / 4;
    size_t tile = ((size_t)blk * Hkv + h) * (size_t)P * d;
    size_t sub = (size_t)(t / 16) * 16 * d;
    int tau = t % 16;
    int n = x / 16, c = x % 16, j = tau / 4, i = tau % 4;
    size_t chunk = ((size_t)(n / R) * 4 + j) * 16 + c;
    return tile + sub + chunk * E + (size_t)((n % R) * 4 + i);
}

static int shape_ok(int dt, int P, int d) {
    if (dt < ORC_F32 || dt > ORC_I8_F16) return 0;
    if (P <= 0 || P % 16 != 0) return 0;
    int E = (int)(16 / elem_size(dt));
    return d > 0 && d % (4 * E) == 0 && d % 16 == 0;
}

/* Value of cache element (blk, h, t, x) of a K (is_v = 0) or V pool. */
static double load_cache(const void* pool, int64_t num_blocks, size_t blk, int h, int t, int x,
                         int Hkv, int P, int d, int dt, int is_v) {
    size_t idx = is_v ? v_index(blk, h, t, x, Hkv, P, d, dt) : k_index(blk, h, t, x, Hkv, P, d, dt);
    if (!is_q8(dt)) return load_elem(pool, idx, dt);
    int8_t q;
    memcpy(&q, (const char*)pool + idx, 1);
    float sc;
    size_t plane = (size_t)num_blocks * Hkv * (size_t)P * d;
    memcpy(&sc, (const char*)pool + plane + (((size_t)blk * Hkv + h) * P + t) * 4, 4);
    return (double)q * (double)sc;
}

/* Quantisation of one row of d values for an INT8 cache (symmetric, one scale per
 * (token, kv head) row, so appending a token never changes earlier ones): with
 * amax = max |x| in fp32, scale = amax / 127 and q = rint(x * (127 / amax)) clamped to
 * [-127, 127], both divisions and the product in fp32 (round to nearest even); a zero row
 * gets scale 0 and q = 0. */
static float quantise_row(const float* x, int d, int8_t* q) {
    float amax = 0.0f;
    for (int i = 0; i < d; ++i) {
        float a = fabsf(x[i]);
        if (a > amax) amax = a;
    }
    if (amax == 0.0f) {
        for (int i = 0; i < d; ++i) q[i] = 0;
        return 0.0f;
    }
    float inv = 127.0f / amax;
    for (int i = 0; i < d; ++i) {
        float r = rintf(x[i] * inv);
        if (r > 127.0f) r = 127.0f;
        if (r < -127.0f) r = -127.0f;
        q[i] = (int8_t)r;
    }
    return amax / 127.0f;
}

/* Exposed for the quantisation pins: quantises `n` rows of d fp32 values. */
int oracle_quantise_rows(const float* x, int n, int d, int8_t* q, float* scales) {
    if (!x || !q || !scales || n < 0 || d <= 0) return ORC_ERR_ARG;
    for (int r = 0; r < n; ++r) scales[r] = quantise_row(x + (size_t)r * d, d, q + (size_t)r * d);
    return ORC_OK;
}

/* Exposed so the tests can check the layout against hand-computed positions. */
int64_t oracle_k_index(int64_t blk, int h, int t, int x, int Hkv, int P, int d, int dt) {
    if (!shape_ok(dt, P, d)) return -1;
    return (int64_t)k_index((size_t)blk, h, t, x, Hkv, P, d, dt);
}
int64_t oracle_v_index(int64_t blk, int h, int t, int x, int Hkv, int P, int d, int dt) {
    if (!shape_ok(dt, P, d)) return -1;
    return (int64_t)v_index((size_t)blk, h, t, x, Hkv, P, d, dt);
}

/* Append ([primer] §2.2; [primer] §4.1): token i goes to slot s = slots[i],
 * block s / P, position s % P, for every kv head and dim; bytes are copied. */
int oracle_kv_append(int dt, int64_t num_blocks, int P, int Hkv, int d,
                     void* kpool, void* vpool, const void* knew, const void* vnew,
                     const int32_t* slots, int64_t n) {
    if (!shape_ok(dt, P, d) || Hkv <= 0 || num_blocks < 0 || n < 0) return ORC_ERR_ARG;
    if (is_q8(dt)) { /* quantise each (token, head) row of K and of V, then store it */
        float* row = (float*)malloc(sizeof(float) * (size_t)d);
        int8_t* q = (int8_t*)malloc((size_t)d);
        if (!row || !q) { free(row); free(q); return ORC_ERR_NOMEM; }
        size_t plane = (size_t)num_blocks * Hkv * (size_t)P * d;
        for (int64_t i = 0; i < n; ++i) {
            int64_t s = slots[i];
            if (s < 0) continue;
            if (s >= num_blocks * (int64_t)P) { free(row); free(q); return ORC_ERR_PRECONDITION; }
            int64_t blk = s / P;
            int t = (int)(s % P);
            for (int h = 0; h < Hkv; ++h)
                for (int is_v = 0; is_v < 2; ++is_v) {
                    const void* src = is_v ? vnew : knew;
                    char* pool = (char*)(is_v ? vpool : kpool);
                    for (int x = 0; x < d; ++x)
                        row[x] = (float)load_elem(src, ((size_t)i * Hkv + h) * d + x, in_dt(dt));
                    float sc = quantise_row(row, d, q);
                    for (int x = 0; x < d; ++x)
                        pool[is_v ? v_index(blk, h, t, x, Hkv, P, d, dt) : k_index(blk, h, t, x, Hkv, P, d, dt)] =
                            (char)q[x];
                    memcpy(pool + plane + (((size_t)blk * Hkv + h) * P + t) * 4, &sc, 4);
                }
        }
        free(row);
        free(q);
        return ORC_OK;
    }
    size_t es = elem_size(dt);
    for (int64_t i = 0; i < n; ++i) {
        int64_t s = slots[i];
        if (s < 0) continue;
        if (s >= num_blocks * (int64_t)P) return ORC_ERR_PRECONDITION;
        int64_t blk = s / P;
        int t = (int)(s % P);
        for (int h = 0; h < Hkv; ++h)
            for (int x = 0; x < d; ++x) {
                size_t src = ((size_t)i * Hkv + h) * d + x;
                memcpy((char*)kpool + k_index(blk, h, t, x, Hkv, P, d, dt) * es,
                       (const char*)knew + src * es, es);
                memcpy((char*)vpool + v_index(blk, h, t, x, Hkv, P, d, dt) * es,
                       (const char*)vnew + src * es, es);
            }
    }
    return ORC_OK;
}

/* Is logical token t (0 <= t < L) attended? Full / window+sinks / page list. */
static int attended(int t, int L, int P, int window, int sinks,
                    const int32_t* pages, int npages) {
    if (pages) {
        for (int k = 0; k < npages; ++k)
            if (pages[k] >= 0 && pages[k] == t / P) return 1;
        return 0;
    }
    if (window > 0 && window < L) return t < sinks || t >= L - window;
    return 1;
}

/* Checks the page-list preconditions of one row: non-negative entries distinct
 * and ascending. */
static int pages_ok(const int32_t* pages, int npages) {
    int last = -1;
    for (int k = 0; k < npages; ++k) {
        if (pages[k] < 0) continue;
        if (pages[k] <= last) return 0;
        last = pages[k];
    }
    return 1;
}

/* Index of the list entry holding logical page p, or -1. */
static int page_entry(const int32_t* pages, int npages, int64_t p) {
    for (int k = 0; k < npages; ++k)
        if (pages[k] >= 0 && pages[k] == p) return k;
    return -1;
}

static int common_args_ok(int dt, int64_t num_blocks, int P, int Hkv, int d, int B, int Hq,
                          int max_blocks, int window, int sinks, const int32_t* page_list,
                          int pps) {
    if (!shape_ok(dt, P, d) || Hkv <= 0 || num_blocks < 0 || B < 0 || Hq <= 0) return 0;
    if (Hq % Hkv != 0 || max_blocks < 0 || sinks < 0) return 0;
    if (page_list && (window > 0 || pps <= 0)) return 0;
    return 1;
}

/* Gathers the logits of one (b, h) over the attended tokens, ascending.
 * Returns the count, or -1 on a precondition violation. */
static int64_t gather_logits(int dt, int64_t num_blocks, int P, int Hkv, int d,
                             const void* kpool, const void* q, int Hq, int b, int h,
                             const int32_t* bt_row, int max_blocks, int L, double scale,
                             int window, int sinks, const int32_t* pages, int npages,
                             double* logits, int64_t* toks) {
    int G = Hq / Hkv;
    int kvh = h / G;
    int64_t cnt = 0;
    for (int t = 0; t < L; ++t) {
        if (!attended(t, L, P, window, sinks, pages, npages)) continue;
        if (t / P >= max_blocks) return -1;
        int64_t blk = bt_row[t / P];
        if (blk < 0 || blk >= num_blocks) return -1;
        double dot = 0.0;
        for (int x = 0; x < d; ++x)
            dot += load_elem(q, ((size_t)b * Hq + h) * d + x, in_dt(dt)) *
                   load_cache(kpool, num_blocks, (size_t)blk, kvh, t % P, x, Hkv, P, d, dt, 0);
        logits[cnt] = scale * dot;
        toks[cnt] = t;
        ++cnt;
    }
    return cnt;
}

/* Decode attention ([TF] formula; [primer] §2.2, §4.1; [OVAL] §3.3 page indices;
 * [primer] §4.3 window). out: [B][Hq][d] doubles; lse: [B][Hq]. */
int oracle_decode_attention(int dt, int64_t num_blocks, int P, int Hkv, int d,
                            const void* kpool, const void* vpool, const void* q,
                            int B, int Hq, const int32_t* block_table, int max_blocks,
                            const int32_t* context_lens, double scale,
                            int window, int sinks, const int32_t* page_list, int pps,
                            double* out, double* lse) {
    if (!common_args_ok(dt, num_blocks, P, Hkv, d, B, Hq, max_blocks, window, sinks,
                        page_list, pps))
        return ORC_ERR_ARG;
    if (scale <= 0.0) scale = 1.0 / sqrt((double)d);
    int G = Hq / Hkv;
    for (int b = 0; b < B; ++b) {
        int L = context_lens[b];
        if (L < 0) return ORC_ERR_PRECONDITION;
        const int32_t* pages = page_list ? page_list + (size_t)b * pps : NULL;
        if (pages && !pages_ok(pages, pps)) return ORC_ERR_PRECONDITION;
        double* logits = (double*)malloc(sizeof(double) * (size_t)(L > 0 ? L : 1));
        int64_t* toks = (int64_t*)malloc(sizeof(int64_t) * (size_t)(L > 0 ? L : 1));
        if (!logits || !toks) { free(logits); free(toks); return ORC_ERR_NOMEM; }
        for (int h = 0; h < Hq; ++h) {
            double* o = out + ((size_t)b * Hq + h) * d;
            int64_t cnt = gather_logits(dt, num_blocks, P, Hkv, d, kpool, q, Hq, b, h,
                                        block_table + (size_t)b * max_blocks, max_blocks, L,
                                        scale, window, sinks, pages, pps, logits, toks);
            if (cnt < 0) { free(logits); free(toks); return ORC_ERR_PRECONDITION; }
            for (int x = 0; x < d; ++x) o[x] = 0.0;
            if (cnt == 0) { lse[(size_t)b * Hq + h] = -INFINITY; continue; }
            double m = logits[0];
            for (int64_t k = 1; k < cnt; ++k) if (logits[k] > m) m = logits[k];
            double z = 0.0;
            for (int64_t k = 0; k < cnt; ++k) z += exp(logits[k] - m);
            int kvh = h / G;
            for (int64_t k = 0; k < cnt; ++k) {
                double w = exp(logits[k] - m);
                int64_t t = toks[k];
                int64_t blk = block_table[(size_t)b * max_blocks + t / P];
                for (int x = 0; x < d; ++x)
                    o[x] += w * load_cache(vpool, num_blocks, (size_t)blk, kvh, (int)(t % P), x, Hkv, P, d, dt, 1);
            }
            for (int x = 0; x < d; ++x) o[x] /= z;
            lse[(size_t)b * Hq + h] = m + log(z);
        }
        free(logits);
        free(toks);
    }
    return ORC_OK;
}

/* Decode-time KV scores ([Novita] §關鍵技術 2: the sparsification score of a token in a
 * head is the sum, over recent queries, of its softmax probability
 * p = exp(q.k - rowmax) / l, which the attention pass already has the rowmax and l for).
 * One decode step contributes its single query per head: for every sequence b, kv head
 * kvh and attended token t,
 *     score[b][kvh][t / block] += sum over the G query heads h of kvh of softmax_h(t),
 * with softmax_h the attention weights of oracle_decode_attention. An entry gathers the
 * scores of `block` consecutive tokens (block = 1: per token; block = the page size: per
 * page). Entries without attended tokens are left as they are, so a caller accumulates over
 * steps by passing the same array again. score: [B][Hkv][stride] doubles; every attended
 * t / block must be < stride. */
int oracle_decode_scores(int dt, int64_t num_blocks, int P, int Hkv, int d,
                         const void* kpool, const void* q, int B, int Hq,
                         const int32_t* block_table, int max_blocks,
                         const int32_t* context_lens, double scale,
                         int window, int sinks, const int32_t* page_list, int pps,
                         double* score, int64_t stride, int block) {
    if (!common_args_ok(dt, num_blocks, P, Hkv, d, B, Hq, max_blocks, window, sinks,
                        page_list, pps) || stride < 0 || block < 1)
        return ORC_ERR_ARG;
    if (scale <= 0.0) scale = 1.0 / sqrt((double)d);
    int G = Hq / Hkv;
    for (int b = 0; b < B; ++b) {
        int L = context_lens[b];
        if (L < 0) return ORC_ERR_PRECONDITION;
        const int32_t* pages = page_list ? page_list + (size_t)b * pps : NULL;
        if (pages && !pages_ok(pages, pps)) return ORC_ERR_PRECONDITION;
        double* logits = (double*)malloc(sizeof(double) * (size_t)(L > 0 ? L : 1));
        int64_t* toks = (int64_t*)malloc(sizeof(int64_t) * (size_t)(L > 0 ? L : 1));
        if (!logits || !toks) { free(logits); free(toks); return ORC_ERR_NOMEM; }
        for (int h = 0; h < Hq; ++h) {
            int64_t cnt = gather_logits(dt, num_blocks, P, Hkv, d, kpool, q, Hq, b, h,
                                        block_table + (size_t)b * max_blocks, max_blocks, L,
                                        scale, window, sinks, pages, pps, logits, toks);
            if (cnt < 0) { free(logits); free(toks); return ORC_ERR_PRECONDITION; }
            if (cnt == 0) continue;
            double m = logits[0];
            for (int64_t k = 1; k < cnt; ++k) if (logits[k] > m) m = logits[k];
            double z = 0.0;
            for (int64_t k = 0; k < cnt; ++k) z += exp(logits[k] - m);
            double* row = score + ((size_t)b * Hkv + h / G) * (size_t)stride;
            for (int64_t k = 0; k < cnt; ++k) {
                int64_t e = toks[k] / block;
                if (e >= stride) { free(logits); free(toks); return ORC_ERR_PRECONDITION; }
                row[e] += exp(logits[k] - m) / z;
            }
        }
        free(logits);
        free(toks);
    }
    return ORC_OK;
}

/* Page selection ([OVAL] §3.3: each step keeps the k pages of highest weight and hands
 * their ids to attention; the config this path is measured on always keeps the page of the
 * newest token). For sequence b with context length L and n = ceil(L / P) pages:
 *   - the weight of page p is sum over h = 0 .. H-1 (in that order) of
 *     scores[b][h][p], accumulated in fp32 (float), so that a caller comparing against a
 *     kernel that sums in the same order sees the same weights bit for bit;
 *   - the newest min(recent, n) pages [n - recent, n) are always taken;
 *   - of the older pages [0, n - recent), the k - recent with the largest weight are
 *     taken; equal weights go to the lower page id;
 *   - out[b] lists the taken ids ascending, then -1 up to k entries.
 * L == 0 gives a row of -1. Preconditions: 0 <= recent <= k, n <= stride, finite scores. */
int oracle_select_pages(const float* scores, int H, int64_t stride, const int32_t* context_lens,
                        int B, int P, int k, int recent, int32_t* out) {
    if (!scores || H <= 0 || stride < 0 || B < 0 || P <= 0 || k <= 0 || recent < 0 ||
        recent > k)
        return ORC_ERR_ARG;
    for (int b = 0; b < B; ++b) {
        int32_t* row = out + (size_t)b * k;
        for (int i = 0; i < k; ++i) row[i] = -1;
        int L = context_lens[b];
        if (L < 0) return ORC_ERR_PRECONDITION;
        int64_t n = ((int64_t)L + P - 1) / P;
        if (n > stride) return ORC_ERR_PRECONDITION;
        if (n == 0) continue;
        int64_t first_recent = n - recent > 0 ? n - recent : 0;
        float* w = (float*)malloc(sizeof(float) * (size_t)(first_recent > 0 ? first_recent : 1));
        char* taken = (char*)calloc((size_t)(first_recent > 0 ? first_recent : 1), 1);
        if (!w || !taken) { free(w); free(taken); return ORC_ERR_NOMEM; }
        for (int64_t p = 0; p < first_recent; ++p) {
            float acc = 0.0f;
            for (int h = 0; h < H; ++h) acc += scores[((size_t)b * H + h) * (size_t)stride + p];
            if (!isfinite(acc)) { free(w); free(taken); return ORC_ERR_PRECONDITION; }
            w[p] = acc;
        }
        /* k - recent rounds of "best remaining page": largest weight, then lowest id */
        int cnt = 0;
        int64_t want = k - recent;
        for (int64_t r = 0; r < want && r < first_recent; ++r) {
            int64_t best = -1;
            for (int64_t p = 0; p < first_recent; ++p) {
                if (taken[p]) continue;
                if (best < 0 || w[p] > w[best]) best = p;  /* ascending p: ties keep the lower id */
            }
            taken[best] = 1;
        }
        for (int64_t p = 0; p < first_recent; ++p)
            if (taken[p]) row[cnt++] = (int32_t)p;
        for (int64_t p = first_recent; p < n; ++p) row[cnt++] = (int32_t)p;
        free(w);
        free(taken);
    }
    return ORC_OK;
}

/* Split partials and their log-sum-exp combination ([Novita] §關鍵技術 2: a
 * partition's running max and sum l are enough to merge it with others).
 * The attended tokens of (b, h) are grouped into aligned 16-token units, which are
 * enumerated and cut into partitions of `units` consecutive enumerated units;
 * partition s gets m_s, l_s and the unnormalised o_s. The enumeration is the one the
 * library's partial call documents: for full and window attention the units t / 16
 * that hold attended tokens, ascending; for a page list every 16-token quarter of
 * every list entry in list order, padding and pages past L included (entry k owns
 * enumerated units k * P/16 .. (k + 1) * P/16 - 1), so a list's partitions depend on
 * the list alone and some of them may be empty. Writes the partials
 * (o_part [B][Hq][S][d], m_part/l_part [B][Hq][S]; empty partitions: m = -inf,
 * l = 0, o = 0) when the pointers are non-NULL, and always the combined
 * out/lse. S = max_splits; more partitions than that is an argument error. */
int oracle_decode_attention_split(int dt, int64_t num_blocks, int P, int Hkv, int d,
                                  const void* kpool, const void* vpool, const void* q,
                                  int B, int Hq, const int32_t* block_table, int max_blocks,
                                  const int32_t* context_lens, double scale,
                                  int window, int sinks, const int32_t* page_list, int pps,
                                  int units, int max_splits,
                                  double* o_part, double* m_part, double* l_part,
                                  double* out, double* lse) {
    if (!common_args_ok(dt, num_blocks, P, Hkv, d, B, Hq, max_blocks, window, sinks,
                        page_list, pps) || units <= 0 || max_splits <= 0)
        return ORC_ERR_ARG;
    if (scale <= 0.0) scale = 1.0 / sqrt((double)d);
    int G = Hq / Hkv;
    double* po = (double*)calloc((size_t)max_splits * d, sizeof(double));
    double* pm = (double*)malloc(sizeof(double) * (size_t)max_splits);
    double* pl = (double*)malloc(sizeof(double) * (size_t)max_splits);
    if (!po || !pm || !pl) { free(po); free(pm); free(pl); return ORC_ERR_NOMEM; }
    int rc = ORC_OK;
    for (int b = 0; b < B && rc == ORC_OK; ++b) {
        int L = context_lens[b];
        const int32_t* pages = page_list ? page_list + (size_t)b * pps : NULL;
        if (L < 0 || (pages && !pages_ok(pages, pps))) { rc = ORC_ERR_PRECONDITION; break; }
        double* logits = (double*)malloc(sizeof(double) * (size_t)(L > 0 ? L : 1));
        int64_t* toks = (int64_t*)malloc(sizeof(int64_t) * (size_t)(L > 0 ? L : 1));
        int64_t* part = (int64_t*)malloc(sizeof(int64_t) * (size_t)(L > 0 ? L : 1));
        if (!logits || !toks || !part) { free(logits); free(toks); free(part); rc = ORC_ERR_NOMEM; break; }
        for (int h = 0; h < Hq && rc == ORC_OK; ++h) {
            int64_t cnt = gather_logits(dt, num_blocks, P, Hkv, d, kpool, q, Hq, b, h,
                                        block_table + (size_t)b * max_blocks, max_blocks, L,
                                        scale, window, sinks, pages, pps, logits, toks);
            if (cnt < 0) { rc = ORC_ERR_PRECONDITION; break; }
            for (int s = 0; s < max_splits; ++s) { pm[s] = -INFINITY; pl[s] = 0.0; }
            memset(po, 0, sizeof(double) * (size_t)max_splits * d);
            /* Each attended token's partition: its enumerated unit / units. */
            int64_t unit_rank = -1, last_unit = -1;
            int kvh = h / G;
            for (int64_t k = 0; k < cnt; ++k) {
                int64_t t = toks[k], u;
                if (pages) {
                    int e = page_entry(pages, pps, t / P);
                    if (e < 0) { rc = ORC_ERR_ARG; break; } /* an attended token lies on a listed page */
                    u = (int64_t)e * (P / 16) + (t % P) / 16;
                } else {
                    if (t / 16 != last_unit) { ++unit_rank; last_unit = t / 16; }
                    u = unit_rank;
                }
                part[k] = u / units;
                if (part[k] >= max_splits) { rc = ORC_ERR_ARG; break; }
            }
            if (rc != ORC_OK) break;
            /* First pass: maxima per partition. */
            for (int64_t k = 0; k < cnt; ++k)
                if (logits[k] > pm[part[k]]) pm[part[k]] = logits[k];
            /* Second pass: sums per partition. */
            for (int64_t k = 0; k < cnt; ++k) {
                int64_t s = part[k];
                double w = exp(logits[k] - pm[s]);
                pl[s] += w;
                int64_t t = toks[k];
                int64_t blk = block_table[(size_t)b * max_blocks + t / P];
                for (int x = 0; x < d; ++x)
                    po[(size_t)s * d + x] +=
                        w * load_cache(vpool, num_blocks, (size_t)blk, kvh, (int)(t % P), x, Hkv, P, d, dt, 1);
            }
            size_t bh = (size_t)b * Hq + h;
            if (o_part) memcpy(o_part + bh * max_splits * d, po, sizeof(double) * (size_t)max_splits * d);
            if (m_part) memcpy(m_part + bh * max_splits, pm, sizeof(double) * (size_t)max_splits);
            if (l_part) memcpy(l_part + bh * max_splits, pl, sizeof(double) * (size_t)max_splits);
            /* Combine: M = max over non-empty partitions; weights exp(m_s - M). */
            double M = -INFINITY;
            for (int s = 0; s < max_splits; ++s) if (pl[s] > 0.0 && pm[s] > M) M = pm[s];
            double* o = out + bh * d;
            for (int x = 0; x < d; ++x) o[x] = 0.0;
            if (M == -INFINITY) { lse[bh] = -INFINITY; continue; }
            double z = 0.0;
            for (int s = 0; s < max_splits; ++s) {
                if (!(pl[s] > 0.0)) continue;
                double w = exp(pm[s] - M);
                z += w * pl[s];
                for (int x = 0; x < d; ++x) o[x] += w * po[(size_t)s * d + x];
            }
            for (int x = 0; x < d; ++x) o[x] /= z;
            lse[bh] = M + log(z);
        }
        free(logits);
        free(toks);
        free(part);
    }
    free(po); free(pm); free(pl);
    return rc;
}

/* Brute force on a contiguous cache: no pool, no block table, no layout.
 * K_log / V_log: [B][Lmax][Hkv][d] logical rows (as a contiguous per-sequence
 * cache would hold them). The token set is built as an explicit list of ranges,
 * and the softmax is the textbook two-pass form in long double. */
int oracle_bruteforce(int dt, const void* K_log, const void* V_log, int Lmax,
                      const void* q, int B, int Hq, int Hkv, int d,
                      const int32_t* context_lens, double scale, int P,
                      int window, int sinks, const int32_t* page_list, int pps,
                      long double* out, long double* lse) {
    if (B < 0 || Hq <= 0 || Hkv <= 0 || Hq % Hkv || d <= 0 || Lmax < 0) return ORC_ERR_ARG;
    if (dt != ORC_F32 && dt != ORC_F16 && dt != ORC_BF16) return ORC_ERR_ARG;
    if (page_list && (P <= 0 || pps <= 0)) return ORC_ERR_ARG;
    long double sc = scale > 0.0 ? (long double)scale : 1.0L / sqrtl((long double)d);
    int G = Hq / Hkv;
    int* idx = (int*)malloc(sizeof(int) * (size_t)(Lmax > 0 ? Lmax : 1));
    long double* lg = (long double*)malloc(sizeof(long double) * (size_t)(Lmax > 0 ? Lmax : 1));
    if (!idx || !lg) { free(idx); free(lg); return ORC_ERR_NOMEM; }
    for (int b = 0; b < B; ++b) {
        int L = context_lens[b];
        if (L < 0 || L > Lmax) { free(idx); free(lg); return ORC_ERR_PRECONDITION; }
        int n = 0;
        if (page_list) {
            for (int k = 0; k < pps; ++k) {
                int p = page_list[(size_t)b * pps + k];
                if (p < 0) continue;
                for (int t = p * P; t < (p + 1) * P && t < L; ++t) idx[n++] = t;
            }
        } else if (window > 0 && window < L) {
            int s_end = sinks < L ? sinks : L;
            int w_begin = L - window > s_end ? L - window : s_end;
            for (int t = 0; t < s_end; ++t) idx[n++] = t;
            for (int t = w_begin; t < L; ++t) idx[n++] = t;
        } else {
            for (int t = 0; t < L; ++t) idx[n++] = t;
        }
        for (int h = 0; h < Hq; ++h) {
            int kvh = h / G;
            long double* o = out + ((size_t)b * Hq + h) * d;
            for (int x = 0; x < d; ++x) o[x] = 0.0L;
            if (n == 0) { lse[(size_t)b * Hq + h] = -INFINITY; continue; }
            for (int k = 0; k < n; ++k) {
                long double acc = 0.0L;
                for (int x = 0; x < d; ++x)
                    acc += (long double)load_elem(q, ((size_t)b * Hq + h) * d + x, dt) *
                           (long double)load_elem(K_log, (((size_t)b * Lmax + idx[k]) * Hkv + kvh) * d + x, dt);
                lg[k] = acc * sc;
            }
            long double m = lg[0];
            for (int k = 1; k < n; ++k) m = lg[k] > m ? lg[k] : m;
            long double z = 0.0L;
            for (int k = 0; k < n; ++k) z += expl(lg[k] - m);
            for (int k = 0; k < n; ++k) {
                long double p = expl(lg[k] - m) / z;
                for (int x = 0; x < d; ++x)
                    o[x] += p * (long double)load_elem(V_log, (((size_t)b * Lmax + idx[k]) * Hkv + kvh) * d + x, dt);
            }
            lse[(size_t)b * Hq + h] = m + logl(z);
        }
    }
    free(idx);
    free(lg);
    return ORC_OK;
}

/* Per-layer memory policy ([Novita] §關鍵技術 1: each layer takes either a full cache or
 * a sliding window over the one paged memory, so window layers need fewer blocks;
 * [primer] §4.3: a window layer keeps only the last W tokens). A window layer attends to
 * the sinks [0, S) and the window [L-W, L) (the reading attention uses). Its block-table
 * row is a ring: the first ceil(S / P) columns hold the sink pages for good, and logical
 * page j past them lives in column sink_pages + (j - sink_pages) mod R, so the block of a
 * page is written over by the page R later. That is safe as long as no two pages that
 * can be attended together share a column: R at least the number of pages that W
 * consecutive tokens can touch. */

static int64_t ring_sink_pages(int sinks, int P) { return sinks > 0 ? ((int64_t)sinks + P - 1) / P : 0; }

/* The most pages W consecutive tokens touch: over the first token's offset o within its
 * page, the pages covering offsets [o, o + W). 0 for W <= 0. */
int oracle_ring_pages(int window, int P) {
    if (window <= 0 || P <= 0) return 0;
    int most = 0;
    for (int o = 0; o < P; ++o) {
        int touched = (o + window + P - 1) / P;
        if (touched > most) most = touched;
    }
    return most;
}

/* Column of logical page j in a ring row. */
int64_t oracle_ring_column(int64_t page, int sinks, int P, int ring_pages) {
    int64_t sp = ring_sink_pages(sinks, P);
    if (page < sp) return page;
    return sp + (page - sp) % ring_pages;
}

/* Plain rows from ring rows: plain[b][j] = ring[b][column(j)] for j < pages, so that
 * block_table[b][t / P] addressing reads what the ring addressing reads. ring: [B][cols];
 * plain: [B][pages]. */
int oracle_ring_expand(const int32_t* ring, int B, int cols, int sinks, int P, int ring_pages,
                       int pages, int32_t* plain) {
    if (B < 0 || cols < 0 || sinks < 0 || P <= 0 || ring_pages <= 0 || pages < 0) return ORC_ERR_ARG;
    if (ring_sink_pages(sinks, P) + ring_pages > cols) return ORC_ERR_ARG;
    for (int b = 0; b < B; ++b)
        for (int j = 0; j < pages; ++j)
            plain[(size_t)b * pages + j] = ring[(size_t)b * cols + oracle_ring_column(j, sinks, P, ring_pages)];
    return ORC_OK;
}

/* Blocks one sequence of L tokens holds in a layer: the distinct table columns its pages
 * [0, ceil(L / P)) use. window <= 0: a full layer (one block per page); otherwise the
 * ring above with R = ring_pages (0: the least safe R). -1 on bad arguments. */
int64_t oracle_policy_blocks(int64_t L, int P, int window, int sinks, int ring_pages) {
    if (L < 0 || P <= 0 || sinks < 0) return -1;
    int64_t pages = (L + P - 1) / P;
    if (window <= 0) return pages;
    if (ring_pages <= 0) ring_pages = oracle_ring_pages(window, P);
    int64_t cols = ring_sink_pages(sinks, P) + ring_pages;
    char* used = (char*)calloc((size_t)cols, 1);
    if (!used) return -1;
    int64_t n = 0;
    for (int64_t j = 0; j < pages; ++j) {
        int64_t c = oracle_ring_column(j, sinks, P, ring_pages);
        if (!used[c]) { used[c] = 1; ++n; }
    }
    free(used);
    return n;
}

/* KV-cache size ([primer] §3.1): 2 (K and V) x batch x layers x heads x head_dim
 * x seq_len x bytes per element; with block_size > 0 the sequence occupies whole
 * blocks, so seq_len is rounded up to a multiple of block_size. */
uint64_t oracle_kv_cache_bytes(int64_t batch, int64_t layers, int64_t heads, int64_t head_dim,
                               int64_t seq_len, int64_t dtype_bytes, int64_t block_size) {
    if (batch < 0 || layers < 0 || heads < 0 || head_dim < 0 || seq_len < 0 || dtype_bytes < 0)
        return 0;
    uint64_t seq = (uint64_t)seq_len;
    if (block_size > 0) seq = (seq + (uint64_t)block_size - 1) / (uint64_t)block_size * (uint64_t)block_size;
    return 2ull * (uint64_t)batch * (uint64_t)layers * (uint64_t)heads * (uint64_t)head_dim * seq *
           (uint64_t)dtype_bytes;
}
