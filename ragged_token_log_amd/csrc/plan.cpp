// Host-side planning for ragged batched token log-probabilities.
//
// Follows [MAX] "MAX Python SDK 中 log_probabilities 模块解析：ragged 批量 Token
// 对数概率的计算图构建与执行":
//   §compute_log_probabilities_ragged -- argument checks at the call boundary;
//   §ragged 数据编排 -- which logits and row offsets the device op reads, and
//     the echo-dependent output counts with their uint32 running-sum offsets;
//   §图支持的最大 top-n / §compute_top 的结果组装 -- the top_n range;
//   §echo 的前置条件 -- echo needs the full logits.
// The chosen token of each row follows [SGL] "logprob、finish reason 与 output
// processing", §input logprob 和 output logprob 来自哪里: a prompt position's
// logits predict the next prompt token, and the last position predicts the
// sampled token.
//
// Nothing here calls HIP, so planning and descriptor building run (and are
// tested) on a machine without a GPU.
#include <cstring>
#include <new>

#include "lp_internal.h"

namespace lp {

void size_workspace(lp_plan &p) {
    p.desc_bytes = align_up(p.out_rows * sizeof(RowDesc), 256);
    p.partial_bytes = p.split > 1 ? p.out_rows * p.split * partial_record_bytes(p.slots) : 0;
    p.workspace_bytes = p.desc_bytes + p.partial_bytes;
}

// Shape of the row kernel (waves per workgroup, chunks in flight per wave,
// segments per row) from the number of rows read, the row length and the
// ranked slots.  Measured on gfx950: 34.6k-row sweeps for the first rule,
// then decode batches of 32..2048 rows at V = 32000, 128256, 151936 and
// 256000, every waves x depth x split timed in interleaved passes.
constexpr uint64_t kManyRows = 1024;
constexpr uint64_t kCUs = 256;
constexpr uint64_t kSplitBelow = 129;   // at most 128 rows: segments (two per row or more)
constexpr uint64_t kLargeKMaxSplit = 4;        // 31+ slots: segments per row at most
constexpr uint32_t kVeryShortRow = 20480;
constexpr uint32_t kShortRow = 65536;
constexpr uint32_t kMinSegment = 32768;
constexpr uint32_t kMinLongSegment = 16000;   // rows longer than kShortRow
constexpr uint32_t kMaxLongSplit = 8;
constexpr uint32_t kMinWideSegment = 24576;   // up to 7 slots: 16 waves from this long

// Segments per row for a batch too small to fill the chip: as many as keep
// the workgroups within one per compute unit (floor, not ceil: a few compute
// units holding two segments double the tail), each at least kMinSegment
// long and within what the merge holds.  Rows longer than kShortRow take
// segments down to kMinLongSegment, up to kMaxLongSplit of them (or as many
// as kMinSegment allows, if more).  At 8-32 rows of 128256, 8 segments take
// 11-12 us against 14 us for 3 at levels 3, and 13-15 against 18 us at
// levels 4; more than 8 lose (8 rows of 256000 at levels 5: 30.6 us in 16
// segments, 24.7 in 8, 31.3 in 7 of 16 waves).
static uint32_t few_rows_split(uint64_t read_rows, uint32_t vocab, uint32_t slots, uint32_t min_split) {
    uint64_t s = kCUs / read_rows;
    uint64_t by_vocab = vocab / kMinSegment;
    if (vocab > kShortRow) {
        const uint64_t fine = vocab / kMinLongSegment;
        const uint64_t most = by_vocab > kMaxLongSplit ? by_vocab : kMaxLongSplit;
        by_vocab = fine < most ? fine : most;
    }
    if (by_vocab < 1) by_vocab = 1;
    if (s > by_vocab) s = by_vocab;
    if (s > max_split_for_slots(slots)) s = max_split_for_slots(slots);
    if (s < min_split) s = min_split;
    return static_cast<uint32_t>(s);
}

static void choose_variant(uint64_t read_rows, uint32_t vocab, uint32_t slots, bool direct,
                           uint32_t *waves, uint32_t *depth, uint32_t *split) {
    // fewest segments that keep each within kMaxSegment (1 for any real vocabulary)
    uint32_t min_split = 1;
    while (segment_length(vocab, min_split) > kMaxSegment) ++min_split;
    *split = min_split;
    *depth = 2;
    const bool many = read_rows >= kManyRows || read_rows == 0;

    if (slots >= 31) {
        // Levels 5 and 6, timed on decode batches of 16-2048 rows at V =
        // 32000 to 256000.  1024 rows or more: 4 waves two deep (within 2 %
        // of the fastest shape).  257-1023 rows: 8 waves one deep (520 rows
        // of 32000: 24.8 against 31.4 us two deep).  129-256: 16 waves one
        // deep (256 rows of 128256 at levels 6: 32.2 against 36.8 us for 8
        // two deep).  At most 128 long rows: 16 waves one deep, up to 4
        // segments a row (16 rows of 151936 at levels 6: 23.3 against 37.3
        // us whole; 8 segments lose to 4 from 63 slots and win by at most 2
        // % at 31).  The seed waits for every wave, so more waves give it
        // more data, and the merge of 4 records stays short.
        if (many) {
            *waves = 4;
            return;
        }
        *depth = 1;
        if (read_rows > kCUs || vocab <= kVeryShortRow) {
            // Two deep, the seed sees twice the row.  Rows found through
            // their descriptors then hold 74 VGPRs, and three workgroups of
            // 8 waves fit a CU (520 rows of 32000 at levels 6: 27.9 against
            // 29.2 us one deep); direct rows also hold the first chunk's
            // copy, 90 VGPRs, and fit two: two deep up to 512 rows (300 rows
            // of 128256 at levels 6: 40.8 against 45.0 us), one deep past
            // it, where workgroups would wait (520 rows of 32000: 33.8
            // against 30.3 us two deep).
            *waves = 8;
            if (vocab > kVeryShortRow && (!direct || read_rows <= 2 * kCUs)) *depth = 2;
            return;
        }
        if (vocab <= kShortRow) {
            // short rows: 8 waves two deep, whole rows (the seed sees two
            // chunks a wave; 4-64 rows of 32000: 12.6-13.6 against
            // 12.8-13.9 us in 4 segments at levels 5, 15.4-16.0 against
            // 15.7-16.9 at levels 6)
            *waves = 8;
            *depth = 2;
            return;
        }
        *waves = 16;
        if (read_rows >= kSplitBelow) return;
        uint64_t s = kCUs / read_rows;
        if (s > kLargeKMaxSplit) s = kLargeKMaxSplit;
        if (s > max_split_for_slots(slots)) s = max_split_for_slots(slots);
        if (s < 1) s = 1;
        *split = s < min_split ? min_split : static_cast<uint32_t>(s);
        return;
    }
    if (many) {
        // 4 waves one chunk deep up to 20K entries per row, 8 waves up to
        // 64K, 16 waves up to 128K, 4 waves two deep beyond (at 34.6k rows:
        // 410 against 435 us for 8 waves at 18992, 202-211 against 291 at
        // 8192; 636 against 655 us for 4 waves at 32000, 2504 against 2551
        // at 128256, 3016 against 3025 at 151936)
        if (vocab <= kVeryShortRow) {
            *waves = 4;
            *depth = 1;
        } else if (vocab <= kShortRow) {
            *waves = 8;
            *depth = 1;
        } else if (vocab <= 131072) {
            *waves = 16;
            *depth = 1;
        } else {
            *waves = 4;
        }
        return;
    }
    if (read_rows > kCUs || vocab <= kVeryShortRow) {
        // more rows than compute units, or rows of at most 20K entries: 8
        // waves one chunk deep (2-8 % ahead of two deep at 320 rows, level
        // at 512; 7-14 % ahead of 16 waves on rows of 8192 and 16000); with
        // at most 3 slots and two rows or more per compute unit, 4 waves
        // (520 rows of 32000 and 128256 at levels 1 and 2: 9-12 % ahead)
        *waves = (slots <= 3 && read_rows >= 2 * kCUs) ? 4 : 8;
        *depth = 1;
        return;
    }
    // One chunk deep from here.  Since every wave ranks at the end (the
    // last wave no longer ranks the workgroup's keys alone), 16 waves gain
    // where 8 two deep used to win.
    *depth = 1;
    if (read_rows >= kSplitBelow) {
        // one row per compute unit at most (129-256 rows): 16 waves (decode,
        // 256 rows of 128256: 23.4 against 23.8 us for 8 waves two deep at
        // levels 3, 24.8 against 26.1 at levels 4); two segments a row would
        // leave more workgroups than compute units (25 against 20 us at 144
        // rows of 128256)
        *waves = 16;
        return;
    }
    // fewer rows still (at most 128): segments (7-40 % ahead of whole rows at
    // 32-96 rows of 151936 or 256000) over 16 waves (at levels 4, 4-64 rows
    // of 128256 and 256000: 5-17 % ahead of 8 waves two deep), or over 8
    // waves at up to 7 slots when a segment is shorter than
    // kMinWideSegment (4 and 16 rows of 128256 in 8 segments of 16032:
    // 10.3 and 11.0 against 10.9 and 11.3 us)
    *split = few_rows_split(read_rows, vocab, slots, min_split);
    *waves = (slots <= 7 && segment_length(vocab, *split) < kMinWideSegment) ? 8 : 16;
}

// Chunks handed to whichever wave of a workgroup frees a buffer first
// (instead of a fixed interleave) when fewer than kManyRows rows are read:
// there each workgroup's last wave decides the launch time, and the waves
// then finish together (decode, 256 rows of 128256: 24.6 -> 23.9 us; 520
// rows of 32000: 16.9 -> 16.9 us).  With many rows the workgroups of a CU
// overlap, their tails do not show, and the fixed order is 0.2-0.5 % faster
// (34637 rows of 151936, 4004 of 256000) and reproducible bit for bit.
static uint32_t dynamic_chunks(const lp_plan &p) {
    return (p.deterministic == 0 && p.read_rows > 0 && p.read_rows < kManyRows) ? 1u : 0u;
}

void shard_shape(const lp_plan &p, uint32_t shard_vocab, uint32_t *waves, uint32_t *depth) {
    if (p.shape_set) {
        *waves = p.waves;
        *depth = p.depth;
        return;
    }
    uint32_t split = 1;   // a shard is one segment of each row
    choose_variant(p.read_rows, shard_vocab, p.slots, p.direct_rows != 0, waves, depth, &split);
}

lp_status build_descriptors(const lp_plan &p, const uint32_t *tokens,
                            const uint32_t *sampled, RowDesc *out) {
    if (p.batch > 0 && sampled == nullptr) return LP_ERR_NULL_ARG;
    bool any_echo = false;
    for (uint32_t n = 0; n < p.batch; ++n) any_echo |= p.echo[n] != 0;
    if (any_echo && tokens == nullptr) return LP_ERR_NULL_ARG;
    const uint64_t total = p.in_off[p.batch];
    if (tokens != nullptr)
        for (uint64_t i = 0; i < total; ++i)
            if (tokens[i] >= p.vocab) return LP_ERR_TOKEN_RANGE;
    for (uint32_t n = 0; n < p.batch; ++n)
        if (sampled[n] >= p.vocab) return LP_ERR_TOKEN_RANGE;

    for (uint32_t n = 0; n < p.batch; ++n) {
        const uint64_t len = p.in_off[n + 1] - p.in_off[n];
        const uint64_t count = p.out_off[n + 1] - p.out_off[n];
        // the rows the op reads: the last `count` rows of the request's range
        const uint64_t src_end = p.has_logits ? p.in_off[n + 1] : uint64_t(n) + 1;
        for (uint64_t k = 0; k < count; ++k) {
            const uint64_t o = p.out_off[n] + k;
            const uint64_t pos = len - count + k;   // prompt position of this row
            RowDesc d;
            d.src_row = static_cast<uint32_t>(src_end - count + k);
            d.chosen = (pos + 1 < len) ? tokens[p.in_off[n] + pos + 1] : sampled[n];
            d.top_n = static_cast<uint32_t>(p.top_n[n]);
            if (d.top_n > 0) d.top_n |= p.top_k[n] << 16;
            uint32_t bits;
            std::memcpy(&bits, &p.temp[n], 4);
            d.temp_bits = bits;
            out[o] = d;
        }
    }
    return LP_OK;
}

}  // namespace lp

extern "C" {

lp_status lp_plan_ragged(uint32_t batch, uint32_t vocab, uint32_t levels,
                         const uint32_t *input_row_offsets, const uint8_t *batch_echo,
                         const int32_t *batch_top_n, int has_logits, uint64_t logits_rows,
                         lp_plan **plan_out, uint32_t *output_row_offsets,
                         uint64_t *out_rows, uint64_t *workspace_bytes) {
    if (plan_out == nullptr) return LP_ERR_NULL_ARG;
    *plan_out = nullptr;
    if (input_row_offsets == nullptr) return LP_ERR_NULL_ARG;
    if (batch > 0 && (batch_echo == nullptr || batch_top_n == nullptr)) return LP_ERR_NULL_ARG;
    if (levels > lp::kMaxLevels) return LP_ERR_UNSUPPORTED;
    const uint32_t columns = lp::columns_for_levels(levels);
    const int32_t max_top_n = int32_t(columns) - 1;
    if (vocab < 1) return LP_ERR_SHAPE;

    // offsets: start at 0, every request non-empty
    if (input_row_offsets[0] != 0) return LP_ERR_OFFSETS;
    for (uint32_t n = 0; n < batch; ++n)
        if (input_row_offsets[n + 1] <= input_row_offsets[n]) return LP_ERR_OFFSETS;
    const uint64_t total = input_row_offsets[batch];
    if (has_logits) {
        if (logits_rows != total) return LP_ERR_SHAPE;
    } else if (logits_rows != batch) {
        return LP_ERR_SHAPE;
    }
    for (uint32_t n = 0; n < batch; ++n) {
        if (batch_top_n[n] < 0) return LP_ERR_TOP_N_NEGATIVE;
        if (batch_top_n[n] > max_top_n) return LP_ERR_TOP_N_TOO_LARGE;
    }
    for (uint32_t n = 0; n < batch; ++n)
        if (batch_echo[n] && !has_logits) return LP_ERR_ECHO_NEEDS_LOGITS;

    lp_plan *p = new (std::nothrow) lp_plan();
    if (p == nullptr) return LP_ERR_NOMEM;
    try {
        p->batch = batch;
        p->vocab = vocab;
        p->levels = levels;
        p->columns = columns;
        p->slots = columns - 1;
        p->has_logits = has_logits ? 1 : 0;
        p->logits_rows = logits_rows;
        p->in_off.assign(input_row_offsets, input_row_offsets + batch + 1);
        p->echo.resize(batch);
        p->top_n.resize(batch);
        p->temp.assign(batch, 1.0f);
        p->top_k.assign(batch, 0u);
        p->out_off.resize(size_t(batch) + 1);
        uint64_t acc = 0, read = 0;
        p->out_off[0] = 0;
        for (uint32_t n = 0; n < batch; ++n) {
            p->echo[n] = batch_echo[n] ? 1 : 0;
            p->top_n[n] = batch_top_n[n];
            const uint64_t count = p->echo[n] ? uint64_t(input_row_offsets[n + 1]) -
                                                    input_row_offsets[n]
                                              : 1;
            acc += count;
            if (batch_top_n[n] > 0) read += count;
            if (acc > 0xFFFFFFFFull) {
                delete p;
                return LP_ERR_SHAPE;   // output offsets are uint32
            }
            p->out_off[n + 1] = static_cast<uint32_t>(acc);
        }
        p->out_rows = acc;
        p->read_rows = read;
        // Output row o reads logits row o when every request is read (top_n >
        // 0) and either none has full logits (request n reads next-token row
        // n) or every request echoes (its output rows are its token rows).
        bool direct = read == acc;
        if (has_logits)
            for (uint32_t n = 0; n < batch && direct; ++n) direct = p->echo[n] != 0;
        p->direct_rows = direct ? 1u : 0u;
    } catch (...) {
        delete p;
        return LP_ERR_NOMEM;
    }
    lp::choose_variant(p->read_rows, vocab, p->slots, p->direct_rows != 0, &p->waves, &p->depth,
                       &p->split);
    p->dynamic_chunks = lp::dynamic_chunks(*p);
    lp::size_workspace(*p);

    if (output_row_offsets != nullptr)
        std::memcpy(output_row_offsets, p->out_off.data(), (size_t(batch) + 1) * 4);
    if (out_rows != nullptr) *out_rows = p->out_rows;
    if (workspace_bytes != nullptr) *workspace_bytes = p->workspace_bytes;
    *plan_out = p;
    return LP_OK;
}

lp_status lp_plan_get_info(const lp_plan *plan, lp_plan_info *info) {
    if (plan == nullptr || info == nullptr) return LP_ERR_NULL_ARG;
    info->batch = plan->batch;
    info->vocab = plan->vocab;
    info->levels = plan->levels;
    info->columns = plan->columns;
    info->out_rows = plan->out_rows;
    info->read_rows = plan->read_rows;
    info->split = plan->split;
    info->waves = plan->waves;
    info->depth = plan->depth;
    info->has_logits = plan->has_logits;
    info->workspace_bytes = plan->workspace_bytes;
    info->direct_rows = plan->direct_rows;
    info->record_words = plan->slots + 2;
    info->deterministic = plan->deterministic;
    return LP_OK;
}

lp_status lp_plan_set_split(lp_plan *plan, uint32_t split) {
    if (plan == nullptr) return LP_ERR_NULL_ARG;
    if (split < 1 || split > lp::max_split_for_slots(plan->slots)) return LP_ERR_UNSUPPORTED;
    if (lp::segment_length(plan->vocab, split) > lp::kMaxSegment) return LP_ERR_UNSUPPORTED;
    plan->split = split;
    lp::size_workspace(*plan);
    return LP_OK;
}

lp_status lp_plan_set_waves(lp_plan *plan, uint32_t waves) {
    if (plan == nullptr) return LP_ERR_NULL_ARG;
    if (waves != 4 && waves != 8 && waves != 16) return LP_ERR_UNSUPPORTED;
    plan->waves = waves;
    plan->shape_set = true;
    return LP_OK;
}

lp_status lp_plan_set_depth(lp_plan *plan, uint32_t depth) {
    if (plan == nullptr) return LP_ERR_NULL_ARG;
    if (depth != 1 && depth != 2) return LP_ERR_UNSUPPORTED;
    plan->depth = depth;
    plan->shape_set = true;
    return LP_OK;
}

lp_status lp_plan_set_deterministic(lp_plan *plan, int deterministic) {
    if (plan == nullptr) return LP_ERR_NULL_ARG;
    plan->deterministic = deterministic ? 1u : 0u;
    plan->dynamic_chunks = lp::dynamic_chunks(*plan);
    return LP_OK;
}

lp_status lp_plan_set_temperature(lp_plan *plan, const float *batch_temperature) {
    if (plan == nullptr) return LP_ERR_NULL_ARG;
    if (batch_temperature == nullptr) {
        plan->temp.assign(plan->batch, 1.0f);
        return LP_OK;
    }
    for (uint32_t n = 0; n < plan->batch; ++n) {
        const float t = batch_temperature[n];
        // within [2^-126, 2^120]: T and the kernels' exponent scale
        // log2(e)/T are normal fp32 numbers, and a logit difference that
        // overflows fp32 (taken as -inf by the kernels) has a weight below
        // e^-256 after the division.  NaN fails both compares.
        if (!(t >= 0x1p-126f && t <= 0x1p120f)) return LP_ERR_TEMPERATURE;
    }
    for (uint32_t n = 0; n < plan->batch; ++n) plan->temp[n] = batch_temperature[n];
    return LP_OK;
}

lp_status lp_plan_set_top_k(lp_plan *plan, const int32_t *batch_top_k) {
    if (plan == nullptr) return LP_ERR_NULL_ARG;
    if (batch_top_k == nullptr) {
        plan->top_k.assign(plan->batch, 0u);
        return LP_OK;
    }
    for (uint32_t n = 0; n < plan->batch; ++n)
        if (batch_top_k[n] < 0 || uint32_t(batch_top_k[n]) > plan->slots) return LP_ERR_TOP_K;
    for (uint32_t n = 0; n < plan->batch; ++n) plan->top_k[n] = uint32_t(batch_top_k[n]);
    return LP_OK;
}

lp_status lp_plan_descriptors(const lp_plan *plan, const uint32_t *tokens,
                              const uint32_t *sampled_tokens, uint32_t *desc_out) {
    if (plan == nullptr || (desc_out == nullptr && plan->out_rows > 0)) return LP_ERR_NULL_ARG;
    return lp::build_descriptors(*plan, tokens, sampled_tokens,
                                 reinterpret_cast<lp::RowDesc *>(desc_out));
}

lp_status lp_assemble_ragged(const lp_plan *plan, const float *lp, const uint32_t *ids,
                             uint32_t *out_tokens, float *out_logprobs, uint32_t *out_counts) {
    if (plan == nullptr) return LP_ERR_NULL_ARG;
    if (plan->out_rows == 0) return LP_OK;
    if (lp == nullptr || ids == nullptr || out_tokens == nullptr || out_logprobs == nullptr ||
        out_counts == nullptr)
        return LP_ERR_NULL_ARG;
    const uint64_t C = plan->columns;
    struct Entry {
        uint32_t token;
        float value;
    };
    std::vector<Entry> e;
    try {
        e.reserve(C + 1);   // a row's entries and the chosen token: no reallocation below
    } catch (...) {
        return LP_ERR_NOMEM;
    }
    for (uint32_t n = 0; n < plan->batch; ++n) {
        const int32_t top_n = plan->top_n[n];
        for (uint64_t o = plan->out_off[n]; o < plan->out_off[n + 1]; ++o) {
            if (top_n == 0) {
                out_counts[o] = 0;
                continue;
            }
            const float *lrow = lp + o * C;
            const uint32_t *irow = ids + o * C;
            e.clear();
            for (uint64_t j = 0; j + 1 < C; ++j)
                if (irow[j] < plan->vocab) e.push_back(Entry{irow[j], lrow[j]});
            // stable insertion sort, descending; a NaN never compares greater,
            // so NaN entries (an all -inf row) keep their order
            for (size_t i = 1; i < e.size(); ++i) {
                const Entry cur = e[i];
                size_t k = i;
                while (k > 0 && cur.value > e[k - 1].value) {
                    e[k] = e[k - 1];
                    --k;
                }
                e[k] = cur;
            }
            if (e.size() > size_t(top_n)) e.resize(size_t(top_n));
            // insertion into a dict keyed by token: a repeated key keeps its
            // first position and takes the later value; the chosen token
            // (last column) goes in last the same way
            e.push_back(Entry{irow[C - 1], lrow[C - 1]});
            size_t kept = 0;
            for (size_t i = 0; i < e.size(); ++i) {
                size_t k = 0;
                while (k < kept && e[k].token != e[i].token) ++k;
                if (k < kept) e[k].value = e[i].value;
                else e[kept++] = e[i];
            }
            e.resize(kept);
            for (size_t k = 0; k < e.size(); ++k) {
                out_tokens[o * C + k] = e[k].token;
                out_logprobs[o * C + k] = e[k].value;
            }
            out_counts[o] = static_cast<uint32_t>(e.size());
        }
    }
    return LP_OK;
}

void lp_plan_destroy(lp_plan *plan) {
    delete plan;
}

const char *lp_status_string(lp_status status) {
    switch (status) {
        case LP_OK: return "LP_OK";
        case LP_ERR_NULL_ARG: return "LP_ERR_NULL_ARG";
        case LP_ERR_OFFSETS: return "LP_ERR_OFFSETS";
        case LP_ERR_SHAPE: return "LP_ERR_SHAPE";
        case LP_ERR_TOP_N_NEGATIVE: return "LP_ERR_TOP_N_NEGATIVE";
        case LP_ERR_TOP_N_TOO_LARGE: return "LP_ERR_TOP_N_TOO_LARGE";
        case LP_ERR_ECHO_NEEDS_LOGITS: return "LP_ERR_ECHO_NEEDS_LOGITS";
        case LP_ERR_TOKEN_RANGE: return "LP_ERR_TOKEN_RANGE";
        case LP_ERR_UNSUPPORTED: return "LP_ERR_UNSUPPORTED";
        case LP_ERR_WORKSPACE: return "LP_ERR_WORKSPACE";
        case LP_ERR_HIP: return "LP_ERR_HIP";
        case LP_ERR_NOMEM: return "LP_ERR_NOMEM";
        case LP_ERR_TEMPERATURE: return "LP_ERR_TEMPERATURE";
        case LP_ERR_TOP_K: return "LP_ERR_TOP_K";
    }
    return "LP_ERR_UNKNOWN";
}

}  // extern "C"
