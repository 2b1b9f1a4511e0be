/* Runs every entry point of the CPU oracle on small random inputs (f32, bf16 and INT8 caches;
 * full, window and page-list modes) so that a build with AddressSanitizer and
 * UndefinedBehaviorSanitizer can check the oracle's memory use. It checks return codes only;
 * the values are pinned elsewhere. Exit status 0 on success. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

int oracle_kv_append(int dt, int64_t num_blocks, int P, int Hkv, int d, void* kpool, void* vpool,
                     const void* knew, const void* vnew, const int32_t* slots, int64_t n);
int oracle_decode_attention(int dt, int64_t num_blocks, int P, int Hkv, int d, const void* kpool,
                            const void* vpool, const void* q, int B, int Hq, const int32_t* block_table,
                            int max_blocks, const int32_t* context_lens, double scale, int window, int sinks,
                            const int32_t* page_list, int pps, double* out, double* lse);
int oracle_decode_scores(int dt, int64_t num_blocks, int P, int Hkv, int d, const void* kpool, const void* q,
                         int B, int Hq, const int32_t* block_table, int max_blocks, const int32_t* context_lens,
                         double scale, int window, int sinks, const int32_t* page_list, int pps, double* score,
                         int64_t stride, int block);
int oracle_decode_attention_split(int dt, int64_t num_blocks, int P, int Hkv, int d, const void* kpool,
                                  const void* vpool, const void* q, int B, int Hq, const int32_t* block_table,
                                  int max_blocks, const int32_t* context_lens, double scale, int window,
                                  int sinks, const int32_t* page_list, int pps, int units, int max_splits,
                                  double* o_part, double* m_part, double* l_part, double* out, double* lse);
int oracle_bruteforce(int dt, const void* K_log, const void* V_log, int Lmax, const void* q, int B, int Hq,
                      int Hkv, int d, const int32_t* context_lens, double scale, int P, int window, int sinks,
                      const int32_t* page_list, int pps, long double* out, long double* lse);
int oracle_select_pages(const float* scores, int H, int64_t stride, const int32_t* context_lens, int B, int P,
                        int k, int recent, int32_t* out);
int oracle_quantise_rows(const float* x, int n, int d, int8_t* q, float* scales);
int oracle_ring_pages(int window, int P);
int oracle_ring_expand(const int32_t* ring, int B, int cols, int sinks, int P, int ring_pages, int pages,
                       int32_t* plain);
int64_t oracle_policy_blocks(int64_t L, int P, int window, int sinks, int ring_pages);
uint64_t oracle_kv_cache_bytes(int64_t batch, int64_t layers, int64_t heads, int64_t head_dim, int64_t seq_len,
                               int64_t dtype_bytes, int64_t block_size);

enum { B = 3, HQ = 4, HKV = 2, D = 64, P = 16, LMAX = 37, NB = 6, STRIDE = 48 };
static const int32_t LENS[B] = {37, 0, 20};
static int failures = 0;

#define CHECK(call)                                                      \
    do {                                                                 \
        int rc_ = (int)(call);                                           \
        if (rc_ != 0) {                                                  \
            fprintf(stderr, "%s:%d: %s returned %d\n", __FILE__, __LINE__, #call, rc_); \
            ++failures;                                                  \
        }                                                                \
    } while (0)

static float frand(void) { return (float)rand() / (float)RAND_MAX * 2.f - 1.f; }
static uint16_t to_bf16(float f) { uint32_t u; memcpy(&u, &f, 4); return (uint16_t)(u >> 16); }

static void run(int dt, int elem_bytes, int pool_row) {
    /* token rows [sum(L)][HKV][D] of the input type, logical rows [B][LMAX][HKV][D] */
    const int ntok = LENS[0] + LENS[1] + LENS[2];
    const int in_bytes = dt == 0 ? 4 : 2;
    unsigned char* knew = calloc((size_t)ntok * HKV * D, in_bytes);
    unsigned char* vnew = calloc((size_t)ntok * HKV * D, in_bytes);
    unsigned char* klog = calloc((size_t)B * LMAX * HKV * D, in_bytes);
    unsigned char* vlog = calloc((size_t)B * LMAX * HKV * D, in_bytes);
    unsigned char* q = calloc((size_t)B * HQ * D, in_bytes);
    for (int i = 0; i < ntok * HKV * D; ++i) {
        float a = frand(), b = frand();
        if (in_bytes == 4) { memcpy(knew + 4 * i, &a, 4); memcpy(vnew + 4 * i, &b, 4); }
        else { uint16_t x = to_bf16(a), y = to_bf16(b); memcpy(knew + 2 * i, &x, 2); memcpy(vnew + 2 * i, &y, 2); }
    }
    for (int i = 0; i < B * HQ * D; ++i) {
        float a = frand();
        if (in_bytes == 4) memcpy(q + 4 * i, &a, 4);
        else { uint16_t x = to_bf16(a); memcpy(q + 2 * i, &x, 2); }
    }
    int32_t bt[B * 3], slots[64];
    int k = 0, blk = 0;
    for (int b = 0; b < B; ++b) {
        for (int j = 0; j < 3; ++j) bt[b * 3 + j] = j * P < LENS[b] ? blk++ : NB - 1;
        for (int t = 0; t < LENS[b]; ++t) {
            slots[k] = bt[b * 3 + t / P] * P + t % P;
            memcpy(klog + (((size_t)b * LMAX + t) * HKV * D) * in_bytes, knew + (size_t)k * HKV * D * in_bytes,
                   (size_t)HKV * D * in_bytes);
            memcpy(vlog + (((size_t)b * LMAX + t) * HKV * D) * in_bytes, vnew + (size_t)k * HKV * D * in_bytes,
                   (size_t)HKV * D * in_bytes);
            ++k;
        }
    }
    const size_t pool_bytes = (size_t)NB * HKV * P * pool_row * elem_bytes;
    void* kpool = calloc(pool_bytes, 1);
    void* vpool = calloc(pool_bytes, 1);
    CHECK(oracle_kv_append(dt, NB, P, HKV, D, kpool, vpool, knew, vnew, slots, ntok));
    double out[B * HQ * D], lse[B * HQ];
    const int32_t pl[B * 2] = {0, 2, -1, -1, 1, -1};
    CHECK(oracle_decode_attention(dt, NB, P, HKV, D, kpool, vpool, q, B, HQ, bt, 3, LENS, 0.0, 0, 0, NULL, 0, out, lse));
    CHECK(oracle_decode_attention(dt, NB, P, HKV, D, kpool, vpool, q, B, HQ, bt, 3, LENS, 0.0, 9, 2, NULL, 0, out, lse));
    CHECK(oracle_decode_attention(dt, NB, P, HKV, D, kpool, vpool, q, B, HQ, bt, 3, LENS, 0.0, 0, 0, pl, 2, out, lse));
    double* score = calloc((size_t)B * HKV * STRIDE, sizeof(double));
    CHECK(oracle_decode_scores(dt, NB, P, HKV, D, kpool, q, B, HQ, bt, 3, LENS, 0.0, 0, 0, NULL, 0, score, STRIDE, 1));
    CHECK(oracle_decode_scores(dt, NB, P, HKV, D, kpool, q, B, HQ, bt, 3, LENS, 0.0, 0, 0, pl, 2, score, STRIDE, P));
    double* op = calloc((size_t)B * HQ * 8 * D, sizeof(double));
    double mp[B * HQ * 8], lp[B * HQ * 8];
    CHECK(oracle_decode_attention_split(dt, NB, P, HKV, D, kpool, vpool, q, B, HQ, bt, 3, LENS, 0.0, 9, 2, NULL, 0,
                                        1, 8, op, mp, lp, out, lse));
    if (dt <= 2) {
        long double bo[B * HQ * D], bl[B * HQ];
        CHECK(oracle_bruteforce(dt, klog, vlog, LMAX, q, B, HQ, HKV, D, LENS, 0.0, P, 9, 2, NULL, 0, bo, bl));
    }
    free(knew); free(vnew); free(klog); free(vlog); free(q); free(kpool); free(vpool); free(score); free(op);
}

int main(void) {
    srand(7);
    run(0, 4, D);       /* fp32 cache */
    run(2, 2, D);       /* bf16 cache */
    run(3, 1, D + 4);   /* INT8 cache with bf16 inputs: data plane then scale plane */
    float sc[2 * 3 * 5];
    for (int i = 0; i < 30; ++i) sc[i] = frand();
    const int32_t cl[2] = {70, 33};
    int32_t sel[2 * 4];
    CHECK(oracle_select_pages(sc, 3, 5, cl, 2, P, 4, 1, sel));
    float x[4 * D];
    int8_t qq[4 * D];
    float scales[4];
    for (int i = 0; i < 4 * D; ++i) x[i] = frand();
    CHECK(oracle_quantise_rows(x, 4, D, qq, scales));
    const int32_t ring[2 * 5] = {0, 1, 2, 3, 4, 5, 6, 7, 8, 9};
    int32_t plain[2 * 12];
    CHECK(oracle_ring_expand(ring, 2, 5, 3, P, oracle_ring_pages(40, P), 12, plain));
    if (oracle_policy_blocks(1000, P, 40, 3, 0) < 0) ++failures;
    if (oracle_kv_cache_bytes(1, 32, 32, 128, 4096, 2, 0) != 2147483648ull) ++failures;
    if (failures) {
        fprintf(stderr, "%d failures\n", failures);
        return 1;
    }
    printf("oracle driver ok\n");
    return 0;
}
