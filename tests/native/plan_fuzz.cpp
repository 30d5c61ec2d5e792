// Randomised driver for the host half of liblogprob (planning, descriptors,
// assembly), meant to run under AddressSanitizer and UndefinedBehaviorSanitizer
// on the CPU.  Every call goes through the C ABI of include/liblogprob.h; the
// inputs mix valid and invalid arguments, and the driver checks the facts the
// header states for each outcome:
//   - on success, output_row_offsets is the running sum of the echo-dependent
//     counts, and the descriptors point inside the logits and the vocabulary;
//   - on error, *plan_out is NULL;
//   - assembly writes at most min(top_n, C - 1) + 1 entries per row and never
//     touches entries past them.
// Prints "ok" and the number of cases that planned, and exits 0 when every
// case holds.
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <random>
#include <vector>

#include "liblogprob.h"

#define CHECK(cond)                                                      \
    do {                                                                 \
        if (!(cond)) {                                                   \
            std::fprintf(stderr, "failed: %s (line %d, case %d)\n", #cond, \
                         __LINE__, case_id);                             \
            return 1;                                                    \
        }                                                                \
    } while (0)

int main(int argc, char **argv) {
    const int cases = argc > 1 ? std::atoi(argv[1]) : 3000;
    std::mt19937_64 rng(12345);
    auto uni = [&](uint64_t lo, uint64_t hi) {   // inclusive
        return lo + rng() % (hi - lo + 1);
    };
    int planned = 0;
    for (int case_id = 0; case_id < cases; ++case_id) {
        const uint32_t batch = uint32_t(uni(0, 9));
        const uint32_t vocab = uint32_t(uni(0, 4) == 0 ? uni(0, 3) : uni(1, 70000));
        const uint32_t levels = uint32_t(uni(0, 7));
        const uint32_t columns = levels > 0 && levels <= 6 ? (1u << levels) : 1u;
        std::vector<uint32_t> off(batch + 1, 0);
        for (uint32_t n = 0; n < batch; ++n) {
            const uint32_t len = uni(0, 40) == 0 ? 0u : uint32_t(uni(1, 30));
            off[n + 1] = off[n] + len;
        }
        if (uni(0, 30) == 0 && batch > 0) off[0] = 1;
        std::vector<uint8_t> echo(batch);
        std::vector<int32_t> top_n(batch);
        for (uint32_t n = 0; n < batch; ++n) {
            echo[n] = uint8_t(uni(0, 1));
            top_n[n] = uni(0, 25) == 0 ? -1 : int32_t(uni(0, columns));   // columns itself is too large
        }
        const int has_logits = int(uni(0, 3) != 0);
        const uint64_t total = off[batch];
        uint64_t logits_rows = has_logits ? total : batch;
        if (uni(0, 30) == 0) logits_rows += 1;

        lp_plan *plan = reinterpret_cast<lp_plan *>(0x1);
        std::vector<uint32_t> out_off(batch + 1, 0xDEADBEEFu);
        uint64_t out_rows = 0, ws = 0;
        const lp_status st = lp_plan_ragged(batch, vocab, levels, off.data(), echo.data(),
                                            top_n.data(), has_logits, logits_rows, &plan,
                                            out_off.data(), &out_rows, &ws);
        if (st != LP_OK) {
            CHECK(plan == nullptr);
            CHECK(std::strlen(lp_status_string(st)) > 0);
            continue;
        }
        CHECK(plan != nullptr);
        ++planned;
        uint64_t acc = 0, read = 0;
        CHECK(out_off[0] == 0);
        for (uint32_t n = 0; n < batch; ++n) {
            const uint64_t count = echo[n] ? uint64_t(off[n + 1] - off[n]) : 1u;
            acc += count;
            if (top_n[n] > 0) read += count;
            CHECK(out_off[n + 1] == acc);
        }
        CHECK(out_rows == acc);
        lp_plan_info info;
        CHECK(lp_plan_get_info(plan, &info) == LP_OK);
        CHECK(info.read_rows == read && info.columns == columns && info.workspace_bytes == ws);
        CHECK(info.record_words == columns + 1);

        // options, valid or not; a refused value leaves the plan as it was
        const uint32_t split = uint32_t(uni(0, 70));
        const lp_status sst = lp_plan_set_split(plan, split);
        CHECK(sst == LP_OK || sst == LP_ERR_UNSUPPORTED);
        (void)lp_plan_set_waves(plan, uint32_t(uni(0, 3) == 0 ? uni(0, 20) : 4u << uni(0, 2)));
        (void)lp_plan_set_depth(plan, uint32_t(uni(0, 3)));
        std::vector<float> temp(batch);
        for (uint32_t n = 0; n < batch; ++n) temp[n] = uni(0, 20) == 0 ? -1.0f : float(uni(1, 400)) / 100.0f;
        const lp_status tst = lp_plan_set_temperature(plan, uni(0, 4) == 0 ? nullptr : temp.data());
        CHECK(tst == LP_OK || tst == LP_ERR_TEMPERATURE);
        std::vector<int32_t> topk(batch);
        for (uint32_t n = 0; n < batch; ++n) topk[n] = int32_t(uni(0, columns + 1)) - (uni(0, 20) == 0 ? 2 : 0);
        const lp_status kst = lp_plan_set_top_k(plan, uni(0, 4) == 0 ? nullptr : topk.data());
        CHECK(kst == LP_OK || kst == LP_ERR_TOP_K);
        CHECK(lp_plan_get_info(plan, &info) == LP_OK);

        // descriptors from exactly-sized token arrays
        std::vector<uint32_t> tokens(total + 1), sampled(batch + 1);
        for (auto &t : tokens) t = vocab > 0 ? uint32_t(uni(0, vocab - 1)) : 0u;
        for (auto &t : sampled) t = vocab > 0 ? uint32_t(uni(0, vocab - 1)) : 0u;
        if (uni(0, 20) == 0 && batch > 0) sampled[0] = vocab;   // out of range
        std::vector<uint32_t> desc(out_rows * 4 + 4, 0xABABABABu);
        const lp_status dst = lp_plan_descriptors(plan, total ? tokens.data() : nullptr,
                                                  sampled.data(), desc.data());
        if (dst == LP_OK) {
            for (uint64_t o = 0; o < out_rows; ++o) {
                CHECK(desc[4 * o] < logits_rows);
                CHECK(desc[4 * o + 1] < vocab);
                CHECK((desc[4 * o + 2] & 0xFFFFu) <= columns - 1);
            }
            CHECK(desc[out_rows * 4] == 0xABABABABu);   // nothing past R rows
        } else {
            CHECK(dst == LP_ERR_TOKEN_RANGE || dst == LP_ERR_NULL_ARG);
        }

        // assembly of random device-shaped rows
        const uint64_t C = columns;
        std::vector<float> lpv(out_rows * C);
        std::vector<uint32_t> ids(out_rows * C);
        for (uint64_t i = 0; i < out_rows * C; ++i) {
            lpv[i] = uni(0, 10) == 0 ? -INFINITY : -float(uni(0, 1000)) / 64.0f;
            ids[i] = uni(0, 5) == 0 ? 0xFFFFFFFFu : uint32_t(uni(0, vocab > 0 ? vocab : 1));
        }
        std::vector<uint32_t> toks(out_rows * C + 1, 0x5A5A5A5Au);
        std::vector<float> vals(out_rows * C + 1, 0.0f);
        std::vector<uint32_t> counts(out_rows + 1, 0x5A5A5A5Au);
        CHECK(lp_assemble_ragged(plan, lpv.data(), ids.data(), toks.data(), vals.data(),
                                 counts.data()) == LP_OK);
        for (uint32_t n = 0; n < batch; ++n)
            for (uint64_t o = out_off[n]; o < out_off[n + 1]; ++o) {
                const uint64_t cap = top_n[n] == 0 ? 0 : uint64_t(top_n[n] < int32_t(C) ? top_n[n] : int32_t(C - 1)) + 1;
                CHECK(counts[o] <= cap);
                for (uint64_t k = counts[o]; k < C; ++k) CHECK(toks[o * C + k] == 0x5A5A5A5Au);
            }
        CHECK(counts[out_rows] == 0x5A5A5A5Au && toks[out_rows * C] == 0x5A5A5A5Au);
        lp_plan_destroy(plan);
    }
    // NULL handling
    int case_id = -1;
    CHECK(lp_plan_ragged(0, 1, 3, nullptr, nullptr, nullptr, 1, 0, nullptr, nullptr, nullptr, nullptr) ==
          LP_ERR_NULL_ARG);
    lp_plan_destroy(nullptr);
    std::printf("ok %d plans\n", planned);
    return 0;
}
