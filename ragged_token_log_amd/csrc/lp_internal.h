// Internal definitions shared by the host plan (plan.cpp) and the device code
// (logprob_kernels.hip).  Not part of the public ABI.
#pragma once

#include <cstddef>
#include <cstdint>
#include <vector>

#include "../../include/liblogprob.h"

namespace lp {

// Output columns per row: 2^levels (one when levels is 0), the last one for
// the chosen token, the others ranked slots; at most 64, one lane each.
constexpr uint32_t kMaxLevels = 6;
constexpr uint32_t kPadId = 0xFFFFFFFFu;
constexpr uint32_t kMaxSplit = 64;
// Keys the merge kernel's one wave holds for a row (16 per lane): the split
// is capped so that split * slots stays within it.
constexpr uint32_t kMaxMergeKeys = 1024;

inline uint32_t columns_for_levels(uint32_t levels) { return levels > 0 ? 1u << levels : 1u; }

inline uint32_t max_split_for_slots(uint32_t slots) {
    if (slots == 0) return kMaxSplit;
    const uint32_t s = kMaxMergeKeys / slots;
    return s < kMaxSplit ? s : kMaxSplit;
}
// Longest vocabulary segment one workgroup streams: its byte range (at most
// 1 GiB) must fit the 32-bit range and offsets of the buffer resource the row
// kernel reads it through.
constexpr uint32_t kMaxSegment = 1u << 28;

// Elements per segment when a row of `vocab` is cut into `split` segments
// (a multiple of 4, so every segment but the first starts 16-byte aligned
// whenever the row does).
inline uint64_t segment_length(uint32_t vocab, uint32_t split) {
    const uint64_t s = (uint64_t(vocab) + split - 1) / split;
    return (s + 3) & ~uint64_t(3);
}

// One output row as the device sees it (16 bytes, one dwordx4 load).
struct RowDesc {
    uint32_t src_row;   // logits row to read (row of `logits` or of next_token_logits)
    uint32_t chosen;    // token whose log-probability goes in the last column
    uint32_t top_n;     // low 16 bits: top_n (0 => padding only, logits not read);
                        // high 16 bits: the top-k front end's k (0 = none)
    uint32_t temp_bits; // fp32 bits of the temperature of the row's request
};
static_assert(sizeof(RowDesc) == 16, "RowDesc is one 16-byte load");

// Partial result of one (row, vocabulary segment or shard), in 8-byte words:
// word 0 holds the segment's running max and scaled sum (two floats), words
// 1..slots its best order keys, descending, word slots + 1 the chosen
// token's logit and a flag set when the segment holds that token.
// Workspace layout: [R descriptors, padded to 256 B][R x split records].
inline uint64_t partial_record_bytes(uint32_t slots) { return 8ull * (uint64_t(slots) + 2); }

inline uint64_t align_up(uint64_t x, uint64_t a) { return (x + a - 1) / a * a; }

}  // namespace lp

struct lp_plan {
    uint32_t batch = 0;
    uint32_t vocab = 0;
    uint32_t levels = 0;
    uint32_t columns = 0;            // 2^levels (1 at levels 0)
    uint32_t slots = 0;              // columns - 1 ranked slots
    uint32_t has_logits = 0;
    uint64_t logits_rows = 0;
    std::vector<uint32_t> in_off;    // B+1
    std::vector<uint32_t> out_off;   // B+1
    std::vector<uint8_t> echo;       // B
    std::vector<int32_t> top_n;      // B
    std::vector<float> temp;         // B: temperature (1 unless set)
    std::vector<uint32_t> top_k;     // B: top-k front end (0 = none unless set)
    uint64_t out_rows = 0;
    uint64_t read_rows = 0;
    uint32_t split = 1;
    uint32_t waves = 4;              // waves per workgroup: 4, 8 or 16
    uint32_t depth = 2;              // chunks in flight per wave: 1 or 2
    bool shape_set = false;          // waves or depth set by the caller
    uint32_t deterministic = 0;      // 1: the caller asked for bit-reproducible sums
    uint32_t dynamic_chunks = 0;     // 1: chunks go to whichever wave is free (see the plan)
    uint32_t direct_rows = 0;        // 1: output row o reads logits row o (all top_n > 0)
    uint64_t desc_bytes = 0;         // R * 16, rounded to 256
    uint64_t partial_bytes = 0;      // R * split * 8 (slots + 2) when split > 1
    uint64_t workspace_bytes = 0;
};

namespace lp {
// Fills `out` (R descriptors) from host token arrays; no HIP calls.
lp_status build_descriptors(const lp_plan &p, const uint32_t *tokens,
                            const uint32_t *sampled, RowDesc *out);
// Recomputes workspace sizes after a split change.
void size_workspace(lp_plan &p);
// Waves and depth for the record kernel of one vocabulary shard of
// `shard_vocab` columns: chosen for that row length, unless the caller set
// the plan's shape.
void shard_shape(const lp_plan &p, uint32_t shard_vocab, uint32_t *waves, uint32_t *depth);
}  // namespace lp
