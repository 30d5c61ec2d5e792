/*
 * liblogprob -- ragged batched token log-probabilities on MI355X (gfx950).
 *
 * For every selected fp32 logits row the library computes, over the whole
 * vocabulary, the log-softmax, the top-n (n <= 2^levels - 1: 7 at the default
 * levels = 3, up to 63 at levels = 6) log-probabilities with their token ids,
 * and the log-probability of the chosen token in one extra slot.
 *
 * Pages the contract follows:
 *   [MAX] "MAX Python SDK 中 log_probabilities 模块解析：ragged 批量 Token 对数概率的
 *         计算图构建与执行"
 *   [SGL] "logprob、finish reason 与 output processing"
 *
 * Layout and conventions shared by every call:
 *   - batch B requests; request n owns token rows [off[n], off[n+1]) of the
 *     full logits ([MAX] §compute_log_probabilities_ragged, the row-offset
 *     argument); L_n = off[n+1] - off[n] >= 1; T = off[B].
 *   - output rows: an echo request gets L_n rows, any other request one row;
 *     output_row_offsets = [0, cumsum(counts)] as uint32 ([MAX] §ragged 数据编排).
 *   - each output row has C = 2^levels columns (8 at levels = 3): columns
 *     0..C-2 hold the top-n log-probabilities in descending order of the raw
 *     fp32 logit (lowest token id first among equal logits, -0.0 == +0.0);
 *     the last column holds the chosen token ([MAX] §log_probabilities_ragged_graph,
 *     §compute_top 的结果组装).  Columns at or beyond min(top_n, V) hold
 *     (-inf, 0xFFFFFFFF); rows of top_n == 0 requests hold that padding in all
 *     C columns and their logits are never read.
 *   - echo row k of request n reads logits row off[n+1] - count_n + k and its
 *     chosen token is the next prompt token tokens[off[n] + p + 1] (p the
 *     prompt position of the row), or the sampled token for the request's last
 *     row ([SGL] §input logprob 和 output logprob 来自哪里).  Without full
 *     logits, request n reads row n of next_token_logits and its chosen token
 *     is sampled_tokens[n].
 *   - every device pointer is caller-allocated device memory; the library
 *     allocates no device memory.  Calls never throw; they return lp_status.
 *   - a logits row must hold no NaN or +inf; -inf entries are allowed and rank
 *     lowest.  An all -inf row yields NaN log-probabilities.
 *   - threads: calls on different plans may run concurrently (the pinned
 *     staging pool behind lp_stage_ragged is shared and locked).  A plan is
 *     not locked: calls that modify it (lp_plan_set_*, lp_plan_destroy) must
 *     not overlap other calls on the same plan; read-only calls on one plan
 *     (staging, launching, assembly, queries) may overlap each other.
 */
#ifndef LIBLOGPROB_H
#define LIBLOGPROB_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct lp_plan lp_plan; /* opaque host object */

typedef enum lp_status {
    LP_OK = 0,
    LP_ERR_NULL_ARG = 1,          /* a required pointer is NULL */
    LP_ERR_OFFSETS = 2,           /* off[0] != 0, or some L_n == 0 (offsets must strictly increase) */
    LP_ERR_SHAPE = 3,             /* row counts or sizes disagree ([MAX] entry assertions) */
    LP_ERR_TOP_N_NEGATIVE = 4,    /* some top_n < 0 ([MAX] §compute_top 的结果组装) */
    LP_ERR_TOP_N_TOO_LARGE = 5,   /* some top_n > 2^levels - 1 ([MAX] §图支持的最大 top-n) */
    LP_ERR_ECHO_NEEDS_LOGITS = 6, /* echo requested without full logits ([MAX] §echo 的前置条件) */
    LP_ERR_TOKEN_RANGE = 7,       /* a token or sampled token >= vocab */
    LP_ERR_UNSUPPORTED = 8,       /* levels > 6, or a split, wave count or depth
                                     the kernels do not provide */
    LP_ERR_WORKSPACE = 9,         /* workspace NULL or smaller than the plan asks */
    LP_ERR_HIP = 10,              /* a HIP runtime call failed; see lp_last_hip_error() */
    LP_ERR_NOMEM = 11,            /* host allocation failed */
    LP_ERR_TEMPERATURE = 12,      /* a temperature outside [2^-126, 2^120] (or NaN) */
    LP_ERR_TOP_K = 13             /* a top-k front end outside 0..2^levels - 1 */
} lp_status;

/* Facts about a plan (all host values). */
typedef struct lp_plan_info {
    uint32_t batch;           /* B */
    uint32_t vocab;           /* V */
    uint32_t levels;          /* 0..6 (3 by default in the bindings) */
    uint32_t columns;         /* C = 2^levels (1 at levels 0, 8 at levels 3) */
    uint64_t out_rows;        /* R = output_row_offsets[B] */
    uint64_t read_rows;       /* output rows whose request has top_n > 0 (logits rows read) */
    uint32_t split;           /* vocabulary segments per row: 1 = one workgroup per row;
                                 > 1 = one workgroup per segment plus a merge kernel */
    uint32_t has_logits;      /* 1 if full logits are given */
    uint32_t waves;           /* waves per workgroup (4, 8 or 16) */
    uint32_t depth;           /* 16-byte-load chunks in flight per wave (1 or 2) */
    uint64_t workspace_bytes; /* device scratch lp_compute_ragged needs */
    uint32_t direct_rows;     /* 1 if output row o reads logits row o for every o (every
                                 request echoes with full logits, or none has full logits,
                                 and every top_n > 0): the kernel then addresses rows
                                 without waiting for their descriptors */
    uint32_t record_words;    /* 8-byte words of one partial record: 2^levels + 1 */
    uint32_t deterministic;   /* 1 if lp_plan_set_deterministic(plan, 1) is in effect */
} lp_plan_info;

/*
 * lp_plan_ragged -- host-only planning (no HIP call, no device memory).
 *
 * [MAX] §compute_log_probabilities_ragged and §ragged 数据编排: validates the
 * per-request arguments, computes the echo-dependent output row counts and
 * their uint32 offsets, and chooses the kernel shape (split, waves, depth)
 * from the number of rows read and the row length.
 *
 *   batch              B (may be 0: nothing to compute)
 *   vocab              V >= 1
 *   levels             0..6: C = 2^levels columns (levels 0: the chosen
 *                      slot alone), top_n <= C - 1
 *   input_row_offsets  host, B+1 uint32, off[0] = 0, strictly increasing
 *   batch_echo         host, B bytes, nonzero = echo
 *   batch_top_n        host, B int32 in [0, C - 1]
 *   has_logits         nonzero if full (T, V) logits will be given; then
 *                      logits_rows must equal T.  Zero: only (B, V)
 *                      next_token_logits exist and no request may echo.
 *   plan_out           receives a new plan; free it with lp_plan_destroy
 *   output_row_offsets host out, B+1 uint32 (may be NULL)
 *   out_rows           host out, R (may be NULL)
 *   workspace_bytes    host out, bytes of device workspace (may be NULL)
 *
 * On error *plan_out is set to NULL and nothing else is written.
 */
lp_status lp_plan_ragged(uint32_t batch, uint32_t vocab, uint32_t levels,
                         const uint32_t *input_row_offsets, const uint8_t *batch_echo,
                         const int32_t *batch_top_n, int has_logits, uint64_t logits_rows,
                         lp_plan **plan_out, uint32_t *output_row_offsets,
                         uint64_t *out_rows, uint64_t *workspace_bytes);

/* Fills *info.  LP_ERR_NULL_ARG if either pointer is NULL. */
lp_status lp_plan_get_info(const lp_plan *plan, lp_plan_info *info);

/*
 * Overrides the plan's split (vocabulary segments per row) and updates its
 * workspace size.  LP_ERR_UNSUPPORTED unless 1 <= split <= min(64,
 * floor(1024 / (C - 1))) and each segment holds at most 2^28 entries (the
 * most one workgroup streams).  The result does not depend on the split
 * beyond fp32 rounding of the log-probabilities: ids and offsets are identical.
 */
lp_status lp_plan_set_split(lp_plan *plan, uint32_t split);

/* Overrides the waves per workgroup (4, 8 or 16); LP_ERR_UNSUPPORTED otherwise.
 * Results do not depend on it beyond fp32 rounding of the log-probabilities.
 * Once waves or depth is set, shard record kernels use the plan's shape too. */
lp_status lp_plan_set_waves(lp_plan *plan, uint32_t waves);

/* Overrides the chunks in flight per wave (1 or 2); LP_ERR_UNSUPPORTED
 * otherwise.  Results are identical for either value. */
lp_status lp_plan_set_depth(lp_plan *plan, uint32_t depth);

/*
 * Reproducibility of the log-probability values (ids, offsets and padding
 * are exact in every mode).  By default (0), a plan that reads fewer than
 * 1024 rows hands the chunks of a row past each wave's first ones to
 * whichever wave of the workgroup frees a buffer first, so that the waves
 * finish together; the fp32 rounding of the row's sum then depends on
 * timing, and two runs may differ in the last bits of a log-probability
 * (about 1e-6 here, well inside the 1e-5 bar against the float64
 * definition).  Plans reading more rows use a fixed assignment and repeat
 * bit for bit.  Nonzero fixes the assignment for every plan: the same inputs
 * and plan shape give bit-identical outputs on every run, at some cost in
 * speed on small batches (decode, 256 rows of 128256: about 0.8 us per
 * launch).  Applies to launches after the call; LP_ERR_NULL_ARG for a NULL
 * plan.
 */
lp_status lp_plan_set_deterministic(lp_plan *plan, int deterministic);

/*
 * Per-request temperature (host, B floats; NULL restores 1 for all).  The
 * log-probabilities of request n become log_softmax(x / T_n) of its rows,
 * the temperature scaling the FlashInfer page describes (its Temperature
 * processor divides the logits by a positive temperature) and that [SGL]
 * §output 从 forward() 到响应对象的完整路径 applies before the softmax whose
 * result the logprobs reuse.  The ranking stays on the raw logits (for T > 0
 * it is the same order).  LP_ERR_TEMPERATURE, with the plan unchanged, if
 * some T_n lies outside [2^-126, 2^120] (or is NaN): inside it T_n and
 * log2(e)/T_n are normal fp32 numbers, and two logits further apart
 * than the fp32 range (whose difference the kernels take as -inf) differ by
 * more than 256 after the division.
 * Applies to descriptors built after the call.
 */
lp_status lp_plan_set_temperature(lp_plan *plan, const float *batch_temperature);

/*
 * Per-request top-k front end (host, B int32; NULL restores 0 = none for all).
 * The FlashInfer page's TopK processor on logits keeps the k highest-scored
 * tokens and masks the others to -inf, and its Softmax then normalises over
 * the kept ones; [SGL] §output 从 forward() 到响应对象的完整路径 names top-k
 * truncation between the temperature scaling and the softmax the logprobs
 * reuse.  With k_n > 0, request n's rows keep exactly the k_n best tokens of
 * the ranking (ties at the boundary go to the lowest ids), their
 * log-probabilities are log_softmax over the kept logits alone (after the
 * temperature), only kept tokens are listed (at most min(top_n, k_n)), and a
 * chosen token outside the kept set gets -inf.  LP_ERR_TOP_K, with the plan
 * unchanged, if some k_n < 0 or k_n > 2^levels - 1 (the kernels rank only
 * that many tokens).  Applies to descriptors built after the call.
 */
lp_status lp_plan_set_top_k(lp_plan *plan, const int32_t *batch_top_k);

/*
 * Host-side row descriptors, for inspection (no HIP call).  Writes R rows of
 * 4 uint32 to desc_out: {logits row read, chosen token, top_n | k << 16 (k the top-k front
 * end; 0 on rows of top_n 0), temperature bits}, in output
 * row order.  tokens: host, T uint32 (may be NULL when no request echoes);
 * sampled_tokens: host, B uint32.  LP_ERR_TOKEN_RANGE if an id >= V.  The
 * fourth word holds the fp32 bits of the row's temperature (the kernels
 * divide by it in fp64 when they write a log-probability).
 */
lp_status lp_plan_descriptors(const lp_plan *plan, const uint32_t *tokens,
                              const uint32_t *sampled_tokens, uint32_t *desc_out);

/*
 * lp_stage_ragged -- builds the row descriptors on the host (tokens and
 * sampled tokens are host arrays, as in [MAX] §compute_log_probabilities_ragged)
 * and enqueues their copy into the device workspace on `stream` (a
 * hipStream_t; NULL = default stream).  The descriptors go through a
 * process-wide pool of pinned host buffers (one per upload in flight, per
 * device): a buffer is reused once the copy from it has finished, so the call
 * neither allocates nor waits in the steady state, and the plan may be
 * destroyed as soon as it returns.
 */
lp_status lp_stage_ragged(const lp_plan *plan, const uint32_t *tokens,
                          const uint32_t *sampled_tokens, void *workspace,
                          uint64_t workspace_bytes, void *stream);

/*
 * lp_launch_ragged -- enqueues the device work on `stream`, reading the
 * descriptors a previous lp_stage_ragged put in `workspace`.
 *
 *   logits             device, (T, V) fp32 row-major contiguous; NULL iff the
 *                      plan has no full logits
 *   next_token_logits  device, (B, V) fp32 row-major; read only when the plan
 *                      has no full logits (may be NULL otherwise)
 *   out_logprobs       device out, (R, C) fp32
 *   out_token_ids      device out, (R, C) uint32
 *   workspace          device, >= workspace_bytes of the plan, 256-byte aligned
 *
 * One kernel launch (two when split > 1).  Enqueue only: no host
 * synchronisation.  Launches that share a workspace must be ordered (same
 * stream): split launches keep partial results there.  Device buffers must stay alive
 * until the stream reaches the end of the enqueued work.
 *
 * It enqueues kernels and nothing else (no copy, no memset, no event), so it
 * may be captured into a HIP graph: the kernels read the logits and the
 * descriptors at replay time, so a caller stages each step's descriptors
 * with lp_stage_ragged (outside the graph, on the replay stream) and replays.
 */
lp_status lp_launch_ragged(const lp_plan *plan, const float *logits,
                           const float *next_token_logits, float *out_logprobs,
                           uint32_t *out_token_ids, void *workspace,
                           uint64_t workspace_bytes, void *stream);

/*
 * lp_compute_ragged -- the descriptors of this call, then the kernels: the
 * results of lp_stage_ragged followed by lp_launch_ragged, with the same
 * arguments and errors.  For plans of at most 262144 output rows the kernels
 * read the descriptors straight from the library's pinned host staging
 * memory and no copy precedes them; the workspace then holds only split
 * records, and its descriptor area is left unwritten (a later
 * lp_launch_ragged on this workspace needs its own lp_stage_ragged).
 * Larger plans stage into the workspace as lp_stage_ragged does.  The
 * staging buffer goes back to the pool once what reads it has ended: the
 * call's last kernel (an event recorded by that kernel's launch) when read
 * in place, else the copy.  In the steady state the call neither allocates
 * nor waits; since it records events, it is not meant to be captured into
 * a HIP graph (lp_launch_ragged is).
 */
lp_status lp_compute_ragged(const lp_plan *plan, const float *logits,
                            const float *next_token_logits, const uint32_t *tokens,
                            const uint32_t *sampled_tokens, float *out_logprobs,
                            uint32_t *out_token_ids, void *workspace,
                            uint64_t workspace_bytes, void *stream);

/*
 * lp_compute_ragged_noalloc -- lp_compute_ragged for callers that cannot
 * allocate memory (code that must not call hipMalloc or a caching allocator,
 * tight serving loops): the same kernels and results, with no workspace
 * argument and no allocation of any kind, device or pinned host.
 *
 * The workspace is a fixed device array of 4 MiB inside the library, one per
 * GPU (each GPU holds it until the process ends), and the descriptors are
 * built in a fixed host array of the same size.  LP_ERR_WORKSPACE, before
 * any HIP call, if the plan's workspace_bytes exceeds 4 MiB (at the default
 * levels, about 262000 output rows without a split).  Other arguments as for
 * lp_compute_ragged; `stream` a hipStream_t (NULL = default stream).
 *
 * Plans of up to 1984 output rows send their descriptors in the arguments
 * of up to 8 launches of a small copy kernel (248 descriptors each), which
 * the runtime takes when it enqueues them: the call waits for nothing.
 * Larger plans copy them from the host array, which is not pinned, so that
 * copy is synchronous: the call returns after the stream has finished its
 * earlier work and the copy, then enqueues the kernels and does not wait
 * for them.  Calls are serialised by a lock while they build and send the
 * descriptors.  Every call on one GPU
 * shares that GPU's array and leaves its last contents there: calls whose
 * kernels overlap on one GPU (on different streams) race; calls on one
 * stream are ordered.
 */
lp_status lp_compute_ragged_noalloc(const lp_plan *plan, const float *logits,
                                    const float *next_token_logits, const uint32_t *tokens,
                                    const uint32_t *sampled_tokens, float *out_logprobs,
                                    uint32_t *out_token_ids, void *stream);

/*
 * lp_assemble_ragged -- host-side result assembly of rows copied back from
 * the device ([MAX] §compute_top 的结果组装; no HIP call).
 *
 * For each output row o (C = columns of the plan), the entries of that
 * row's top-log-probability dict, in insertion order:
 *   1. the ranked columns 0..C-2 whose token id is < V (padding dropped),
 *      sorted by log-probability, descending (stable: equal values keep
 *      their column order), truncated to the request's top_n;
 *   2. the chosen token of the last column: appended when absent, else its
 *      value overwrites the existing entry in place.
 * Rows of requests with top_n == 0 get no entries (the request's result is
 * None on the page).  The request's token log-probabilities are the last
 * column of its rows.
 *
 *   lp, ids       host, (R, C) fp32 / uint32 as written by lp_launch_ragged
 *   out_tokens    host out, (R, C) uint32: row o's entries at [o*C, o*C + n_o)
 *   out_logprobs  host out, (R, C) fp32, matching out_tokens
 *   out_counts    host out, R uint32: n_o (at most min(top_n, C-1) + 1)
 * Entries past n_o are left as they were.  LP_ERR_NULL_ARG if a pointer is
 * NULL while R > 0.
 */
lp_status lp_assemble_ragged(const lp_plan *plan, const float *lp, const uint32_t *ids,
                             uint32_t *out_tokens, float *out_logprobs, uint32_t *out_counts);

/*
 * Vocabulary-sharded logits (a tensor-parallel LM head, where each GPU holds
 * the logits of one vocabulary range: the "TP worker" of [SGL] §output 从
 * forward() 到响应对象的完整路径).  Each shard reduces its columns of every
 * read row to one partial record; after the records of all shards are
 * gathered, lp_merge_shards writes the rows -- the same results as the
 * unsharded computation over the whole vocabulary (ids bit for bit).
 *
 * A record is record_words (lp_plan_info) 8-byte words: (max, scaled sum)
 * of the shard's part of the row, its best 2^levels - 1 order keys with
 * global token ids, and the chosen token's logit with a flag set when the
 * shard holds the chosen token.  Record words are opaque to the caller.
 *
 * lp_shard_records -- records of shard [vocab_begin, vocab_begin +
 * shard_vocab) of the plan's vocabulary.
 *   shard_logits / shard_next_token_logits  device, rows of shard_vocab fp32
 *     (the shard's columns only; row layout and which one is read as in
 *     lp_launch_ragged)
 *   records    device out, R * record_words 8-byte words, row-major by output
 *              row (rows of top_n == 0 requests are not written)
 *   workspace  as for lp_launch_ragged, after lp_stage_ragged
 * LP_ERR_SHAPE if the range does not fit in [0, V); one kernel launch,
 * whose workgroup shape is chosen for a row of shard_vocab entries unless the
 * caller set the plan's waves or depth.
 *
 * lp_merge_shards -- merges, for every output row, num_shards records laid
 * out shard-major: record (s, o) at word (s * R + o) * record_words of
 * `records` (device).  The shards must cover [0, V) once each; a row whose
 * chosen token no shard holds gets a NaN last column.  LP_ERR_UNSUPPORTED if
 * num_shards is not in 1..64 or num_shards * (2^levels - 1) > 1024.  One
 * kernel launch; outputs as for lp_launch_ragged.
 */
lp_status lp_shard_records(const lp_plan *plan, uint32_t vocab_begin, uint32_t shard_vocab,
                           const float *shard_logits, const float *shard_next_token_logits,
                           uint64_t *records, void *workspace, uint64_t workspace_bytes,
                           void *stream);

lp_status lp_merge_shards(const lp_plan *plan, uint32_t num_shards, const uint64_t *records,
                          float *out_logprobs, uint32_t *out_token_ids, void *workspace,
                          uint64_t workspace_bytes, void *stream);

/* Frees the plan (host memory only; it never waits for the device).  NULL
 * is a no-op. */
void lp_plan_destroy(lp_plan *plan);

/* Static text for a status ("LP_OK", "LP_ERR_SHAPE", ...). */
const char *lp_status_string(lp_status status);

/* The hipError_t of the last failing HIP call in this thread (0 if none). */
int lp_last_hip_error(void);

/*
 * Measurement aid: a plain streaming read of `rows` rows of row_len fp32
 * values (device, contiguous, 16-byte aligned, row_len a multiple of 4; each
 * value read once with nontemporal 16-byte loads, one workgroup per row)
 * that writes each row's sum to partial_out[rows] (device).  It gives the
 * practical HBM read ceiling on the same bytes and row shape the
 * log-probability kernels stream.  LP_ERR_UNSUPPORTED for a misaligned x or
 * row_len.
 */
lp_status lp_bench_stream_read(const float *x, uint32_t rows, uint32_t row_len, float *partial_out,
                               void *stream);

/*
 * Measurement aid: the same plain read in another launch shape, to sweep
 * what the memory system gives a row shape.  Each row is read by `segments`
 * (1..64) workgroups of `threads` (256, 512 or 1024) threads, each taking one
 * contiguous share of the row's float4s with `loads` (1, 2, 4 or 8)
 * nontemporal 16-byte loads in flight per thread; workgroup row * segments +
 * seg writes its share's sum to partial_out[rows * segments] (device).
 * LP_ERR_UNSUPPORTED for a misaligned x or row_len, a shape outside those
 * values, or rows * segments >= 2^31.
 */
lp_status lp_bench_stream_read_shape(const float *x, uint32_t rows, uint32_t row_len,
                                     uint32_t segments, uint32_t threads, uint32_t loads,
                                     float *partial_out, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* LIBLOGPROB_H */
