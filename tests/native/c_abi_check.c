/* A plain C11 caller of liblogprob's host entry points (no GPU needed):
 * plans a small ragged batch, reads the plan's facts and descriptors, runs
 * the host assembly on hand-made outputs, and checks the error statuses.
 * Prints "ok" and returns 0 when every check holds. */
#include <math.h>
#include <stdio.h>
#include <string.h>

#include "liblogprob.h"

#define CHECK(cond)                                                      \
    do {                                                                 \
        if (!(cond)) {                                                   \
            printf("failed: %s (line %d)\n", #cond, __LINE__);           \
            return 1;                                                    \
        }                                                                \
    } while (0)

int main(void) {
    /* requests of 3 and 2 prompt tokens; the first echoes, the second not */
    const uint32_t offsets[3] = {0, 3, 5};
    const uint8_t echo[2] = {1, 0};
    const int32_t top_n[2] = {2, 0};
    lp_plan *plan = NULL;
    uint32_t out_off[3];
    uint64_t out_rows = 0, ws_bytes = 0;
    CHECK(lp_plan_ragged(2, 10, 3, offsets, echo, top_n, 1, 5, &plan, out_off, &out_rows,
                         &ws_bytes) == LP_OK);
    CHECK(plan != NULL);
    CHECK(out_rows == 4 && out_off[0] == 0 && out_off[1] == 3 && out_off[2] == 4);
    CHECK(ws_bytes >= 4 * 16);

    lp_plan_info info;
    CHECK(lp_plan_get_info(plan, &info) == LP_OK);
    CHECK(info.batch == 2 && info.vocab == 10 && info.columns == 8 && info.out_rows == 4);
    CHECK(info.read_rows == 3 && info.record_words == 9);

    /* descriptors: echo rows 0..2 of request 0 predict tokens 1, 2 and the
     * sampled token; request 1 (top_n 0) keeps a row of padding */
    const uint32_t tokens[5] = {4, 5, 6, 7, 8};
    const uint32_t sampled[2] = {9, 3};
    uint32_t desc[4 * 4];
    CHECK(lp_plan_descriptors(plan, tokens, sampled, desc) == LP_OK);
    CHECK(desc[0] == 0 && desc[1] == 5 && desc[2] == 2);
    CHECK(desc[4] == 1 && desc[5] == 6);
    CHECK(desc[8] == 2 && desc[9] == 9);
    CHECK(desc[12 + 2] == 0);
    float temp_word;
    memcpy(&temp_word, &desc[3], 4);
    CHECK(temp_word == 1.0f);

    /* temperature and top-k front end in the descriptors */
    const float temps[2] = {0.5f, 2.0f};
    CHECK(lp_plan_set_temperature(plan, temps) == LP_OK);
    const int32_t ks[2] = {1, 0};
    CHECK(lp_plan_set_top_k(plan, ks) == LP_OK);
    CHECK(lp_plan_descriptors(plan, tokens, sampled, desc) == LP_OK);
    memcpy(&temp_word, &desc[3], 4);
    CHECK(temp_word == 0.5f && desc[2] == (2u | (1u << 16)));
    const int32_t bad_k[2] = {8, 0};
    CHECK(lp_plan_set_top_k(plan, bad_k) == LP_ERR_TOP_K);
    const float bad_t[2] = {0.0f, 1.0f};
    CHECK(lp_plan_set_temperature(plan, bad_t) == LP_ERR_TEMPERATURE);

    /* host assembly: row 0 lists ids 7 and 2 (padding after), chosen 5 */
    float lp[4 * 8];
    uint32_t ids[4 * 8];
    for (int i = 0; i < 4 * 8; ++i) {
        lp[i] = -INFINITY;
        ids[i] = 0xFFFFFFFFu;
    }
    lp[0] = -0.5f; ids[0] = 7;
    lp[1] = -1.5f; ids[1] = 2;
    lp[7] = -3.0f; ids[7] = 5;
    uint32_t toks[4 * 8], counts[4];
    float vals[4 * 8];
    CHECK(lp_assemble_ragged(plan, lp, ids, toks, vals, counts) == LP_OK);
    CHECK(counts[0] == 3 && toks[0] == 7 && toks[1] == 2 && toks[2] == 5);
    CHECK(vals[0] == -0.5f && vals[2] == -3.0f);
    CHECK(counts[3] == 0);

    /* errors at planning time */
    lp_plan *bad = NULL;
    const int32_t neg[2] = {-1, 0};
    CHECK(lp_plan_ragged(2, 10, 3, offsets, echo, neg, 1, 5, &bad, NULL, NULL, NULL) ==
          LP_ERR_TOP_N_NEGATIVE && bad == NULL);
    const uint8_t echo_both[2] = {1, 1};
    CHECK(lp_plan_ragged(2, 10, 3, offsets, echo_both, top_n, 0, 2, &bad, NULL, NULL, NULL) ==
          LP_ERR_ECHO_NEEDS_LOGITS);
    CHECK(strcmp(lp_status_string(LP_ERR_TOP_K), "LP_ERR_TOP_K") == 0);

    lp_plan_destroy(plan);
    lp_plan_destroy(NULL);
    printf("ok\n");
    return 0;
}
