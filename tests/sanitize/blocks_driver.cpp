// Drives the host block manager (per-layer memory policy) through a random walk of appends,
// releases, table reads and rejected calls, so that a build with AddressSanitizer and
// UndefinedBehaviorSanitizer can check its memory use; blocks in use are checked against
// pkv_policy_blocks along the way. Exit status 0 on success.
#include <cstdio>
#include <random>
#include <vector>

#include "pagedkv.h"

int main() {
    const int P = 16, S = 8, MAXP = 40;
    pkv_layer_group g[3] = {{0, 0, 0, 200}, {40, 3, 0, 40}, {23, 20, 5, 60}};
    pkv_block_manager* bm = nullptr;
    if (pkv_bm_create(P, S, MAXP, g, 3, &bm) != PKV_OK) return 1;
    std::mt19937 rng(11);
    std::vector<long long> len(S, 0);
    int failures = 0;
    for (int it = 0; it < 2000; ++it) {
        const int op = (int)(rng() % 10);
        if (op == 0) {
            const int s = (int)(rng() % S);
            if (pkv_bm_release(bm, s) != PKV_OK) ++failures;
            len[s] = 0;
        } else {
            int32_t ids[3], cnt[3];
            const int n = 1 + (int)(rng() % 3);
            for (int i = 0; i < n; ++i) {
                ids[i] = (int32_t)(rng() % (S + 1)) - (i == 2 ? 1 : 0);  // out of range or repeated now and then
                cnt[i] = op < 4 ? (int32_t)(rng() % 50) : 1;
            }
            long long total = 0;
            for (int i = 0; i < n; ++i) total += cnt[i];
            std::vector<int32_t> slots((size_t)(3 * (total > 0 ? total : 1)));
            int32_t lens[3];
            const pkv_status st = pkv_bm_append(bm, ids, cnt, n, slots.data(), lens);
            if (st == PKV_OK)
                for (int i = 0; i < n; ++i) len[ids[i]] += cnt[i];
            else if (st != PKV_ERR_SHAPE && st != PKV_ERR_NO_BLOCKS)
                ++failures;
        }
        for (int gi = 0; gi < 3; ++gi) {
            long long want = 0;
            for (int s = 0; s < S; ++s) want += pkv_policy_blocks(len[s], P, g[gi].window, g[gi].num_sinks, g[gi].ring_pages);
            if (pkv_bm_blocks_in_use(bm, gi) != want) ++failures;
            std::vector<int32_t> ids(S), table((size_t)S * pkv_bm_table_cols(bm, gi));
            for (int s = 0; s < S; ++s) ids[s] = s;
            if (pkv_bm_block_tables(bm, gi, ids.data(), S, table.data()) != PKV_OK) ++failures;
        }
    }
    pkv_bm_destroy(bm);
    if (failures) {
        std::fprintf(stderr, "%d failures\n", failures);
        return 1;
    }
    std::printf("block manager driver ok\n");
    return 0;
}
