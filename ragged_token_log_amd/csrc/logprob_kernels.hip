// Device code and launch glue for ragged batched token log-probabilities on
// CDNA4 (gfx950, wave64).
//
// What is computed follows [MAX] "MAX Python SDK 中 log_probabilities 模块解析：
// ragged 批量 Token 对数概率的计算图构建与执行" (§log_probabilities_ragged_graph:
// per output row, 2^levels - 1 ranked slots plus one slot for the chosen
// token; §图支持的最大 top-n: top_n <= 2^levels - 1) and [SGL] "logprob、finish
// reason 与 output processing" (§logprob 的数值形态: a logprob is log p, so
// <= 0), with the FlashInfer page's Temperature and TopK-then-Softmax as
// options.  The pages keep the candidates in a min-heap; this file does not.
// On gfx950 the work is an HBM stream with a few VALU ops per element, so the
// design aims at reading each logit exactly once with 16-byte loads and doing
// as little per element as possible:
//
//  * Each row (or row segment, or vocabulary shard) is one workgroup of 4, 8
//    or 16 waves.  Waves take interleaved chunks of 64 lanes x kU float4,
//    read with nontemporal buffer loads, one or two chunks in flight per
//    wave (two buffers taken in turn at 31+ slots with 16 waves one deep).
//    Per chunk a lane reduces its 16 values to a chunk max and updates
//    a running (m, s) with s = sum 2^((x - m) log2(e) / T), the subtraction
//    first.
//  * Ranking uses a 64-bit order key: the fp32 bits mapped to an unsigned
//    order (with -0.0 folded onto +0.0) in the high word, the complemented
//    token id in the low word.  A larger key is a better (value, id) pair, so
//    ties go to the lowest id and every merge uses one total order.
//  * Each wave keeps its K best keys sorted across lanes 0..K-1 and filters
//    its chunks against a bound T (its own K-th key, a workgroup maximum of
//    such keys in LDS, and a seed from the first chunks' maxima; from 31
//    slots also the waves' published keys).  A chunk whose lane maxima stay
//    below T costs one compare; the few columns that beat it enter their
//    keys one at a time, or at 63 slots are gathered and merged in bulk.
//  * The waves' lists and (max, sum) pairs meet in LDS; the waves rank the
//    keys against all the lists while the last wave combines the pairs, and
//    wave 0 writes lp = (x - M) / T - ln S for the K best and for the chosen
//    token, or, for segments and shards, a record of (M, S, K keys, chosen
//    logit) that a second kernel (one wave per row) merges.
//
// No MFMA: there is no contraction here.
#include <hip/hip_runtime.h>
#include <hip/hip_ext.h>

#include <algorithm>
#include <cstdint>
#include <cstring>
#include <deque>
#include <memory>
#include <mutex>
#include <new>
#include <type_traits>
#include <vector>

#include "lp_internal.h"

namespace lp {
namespace dev {

constexpr int kWave = 64;
constexpr int kU = 4;                // float4 loads per lane per chunk
constexpr int kChunkF4 = kWave * kU; // float4 per wave-chunk (1024 elements)
constexpr double kLog2eF64 = 1.4426950408889634;   // log2(e)

// ------------------------------------------------------------------ order keys

__device__ __forceinline__ uint64_t order_key(float v, uint32_t id) {
    uint32_t u = __float_as_uint(v);
    if (u == 0x80000000u) u = 0u;  // -0.0 ranks equal to +0.0
    const uint32_t hi = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
    return (uint64_t(hi) << 32) | uint64_t(~id);
}

__device__ __forceinline__ float key_value(uint64_t k) {
    const uint32_t hi = uint32_t(k >> 32);
    const uint32_t u = (hi & 0x80000000u) ? (hi & 0x7FFFFFFFu) : ~hi;
    return __uint_as_float(u);
}

__device__ __forceinline__ uint32_t key_id(uint64_t k) { return ~uint32_t(k); }

__device__ __forceinline__ uint64_t umax64(uint64_t a, uint64_t b) { return a > b ? a : b; }

// ------------------------------------------------------------------ wave helpers
//
// Wave-wide reductions use DPP inside each row of 16 lanes (swap neighbours,
// swap pairs, mirror half-rows, mirror rows) and then read the four row
// results with readlane, so no step goes through the LDS crossbar.

constexpr int kDppXor1 = 0xB1;        // quad_perm(1,0,3,2)
constexpr int kDppXor2 = 0x4E;        // quad_perm(2,3,0,1)
constexpr int kDppHalfMirror = 0x141; // lane i <-> 7-i within 8
constexpr int kDppMirror = 0x140;     // lane i <-> 15-i within 16

template <int kCtrl>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t v) {
    return uint32_t(__builtin_amdgcn_update_dpp(0, int(v), kCtrl, 0xF, 0xF, false));
}
template <int kCtrl>
__device__ __forceinline__ float dpp_f32(float v) {
    return __uint_as_float(dpp_u32<kCtrl>(__float_as_uint(v)));
}

__device__ __forceinline__ uint32_t readlane_u32(uint32_t v, int lane) {
    return uint32_t(__builtin_amdgcn_readlane(int(v), lane));
}
__device__ __forceinline__ float readlane_f32(float v, int lane) {
    return __uint_as_float(readlane_u32(__float_as_uint(v), lane));
}
__device__ __forceinline__ uint64_t readlane_u64(uint64_t v, int lane) {
    return (uint64_t(readlane_u32(uint32_t(v >> 32), lane)) << 32) | readlane_u32(uint32_t(v), lane);
}

__device__ __forceinline__ uint64_t uniform64(uint64_t v) { return readlane_u64(v, 0); }

// The minimum over the first kN (<= 16) lanes' values, all lanes of the
// first row of 16 taking part (lanes kN..15 must hold ~0).
template <int kN>
__device__ __forceinline__ uint64_t first_lanes_min_u64(uint64_t v) {
    static_assert(kN >= 2 && kN <= 16, "within one row");
    auto step = [&](auto ctrl) __attribute__((always_inline)) {
        constexpr int kCtrl = decltype(ctrl)::value;
        const uint64_t o = (uint64_t(dpp_u32<kCtrl>(uint32_t(v >> 32))) << 32) | dpp_u32<kCtrl>(uint32_t(v));
        v = o < v ? o : v;
    };
    step(std::integral_constant<int, kDppXor1>{});
    if constexpr (kN > 2) step(std::integral_constant<int, kDppXor2>{});
    if constexpr (kN > 4) step(std::integral_constant<int, kDppHalfMirror>{});
    if constexpr (kN > 8) step(std::integral_constant<int, kDppMirror>{});
    return readlane_u64(v, 0);
}

__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
    v = max(v, dpp_u32<kDppXor1>(v));
    v = max(v, dpp_u32<kDppXor2>(v));
    v = max(v, dpp_u32<kDppHalfMirror>(v));
    v = max(v, dpp_u32<kDppMirror>(v));
    return max(max(readlane_u32(v, 0), readlane_u32(v, 16)),
               max(readlane_u32(v, 32), readlane_u32(v, 48)));
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// The exponent scale log2(e) / temperature of every sum e^((x - m) /
// temperature) = 2^((x - m) * scale), rounded once from fp64.  The row and
// merge kernels both take it from here, so partial sums scaled in one and
// combined in the other agree.
__device__ __forceinline__ float exp2_scale(float temp) {
    return float(kLog2eF64 / double(temp));
}

// Orders this wave's LDS accesses around an LDS counter: the workgroup-scope
// fences restricted to LDS wait only for outstanding LDS operations, never
// for the wave's in-flight global loads.
__device__ __forceinline__ void lds_release() { __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local"); }
__device__ __forceinline__ void lds_acquire() { __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local"); }

// A relaxed read of an LDS word that other waves update atomically.  It stays
// an LDS access (a volatile read through a generic pointer would become a flat
// access, whose wait also drains the wave's in-flight global loads).
__device__ __forceinline__ uint64_t lds_load_relaxed(const uint64_t *p) {
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
}

// Logits are read exactly once: nontemporal 16-byte loads (the `nt` form of
// buffer_load_dwordx4) stream them without displacing reusable cache lines;
// on gfx950 they sustain ~13% more HBM bandwidth than plain loads here.
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

// s_waitcnt immediate on gfx9-family parts: vmcnt(0), expcnt(7), lgkmcnt(15)
constexpr int kWaitVmcnt0 = 0x0F70;

constexpr int kBufferWord3 = 0x00020000;  // raw buffer, 32-bit data format (gfx9 family)
constexpr int kAuxNontemporal = 2;         // cache-policy bit of the buffer load: nt

struct StreamRange {
    __amdgpu_buffer_rsrc_t rsrc;
};

// A raw buffer over `bytes` bytes starting at p (16-byte aligned); the range
// fits 31 bits because a segment holds at most 2^29 elements.
__device__ __forceinline__ StreamRange make_stream_range(const float *p, uint32_t bytes) {
    return StreamRange{__builtin_amdgcn_make_buffer_rsrc(const_cast<float *>(p), 0, int(bytes), kBufferWord3)};
}

// 16 bytes at byte offset off; zeros, with no memory access, past the range.
__device__ __forceinline__ f32x4 stream_load(const StreamRange &r, uint32_t off) {
    return __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(r.rsrc, off, 0, kAuxNontemporal));
}

// (m, s) with s = sum e^(x - m): merge (m2, s2) into (m, s).  A max of -inf
// (nothing finite seen) contributes nothing and never forms -inf - -inf.
// Symmetric in its two operands, so both lanes of a butterfly agree bit for bit.
// c = log2(e) / temperature: every sum is of e^((x - m) / temperature)
__device__ __forceinline__ void lse_merge(float &m, float &s, float m2, float s2, float c) {
    const float M = fmaxf(m, m2);
    const float Ms = (M == -INFINITY) ? 0.0f : M;
    s = s * fast_exp2((m - Ms) * c) + s2 * fast_exp2((m2 - Ms) * c);
    m = M;
}

template <int kCtrl>
__device__ __forceinline__ void lse_dpp_step(float &m, float &s, float c) {
    const float m2 = dpp_f32<kCtrl>(m);
    const float s2 = dpp_f32<kCtrl>(s);
    lse_merge(m, s, m2, s2, c);
}

// Every lane ends with the wave's (m, s), merged in a fixed order.
__device__ __forceinline__ void wave_lse(float &m, float &s, float c) {
    lse_dpp_step<kDppXor1>(m, s, c);
    lse_dpp_step<kDppXor2>(m, s, c);
    lse_dpp_step<kDppHalfMirror>(m, s, c);
    lse_dpp_step<kDppMirror>(m, s, c);
    float M = readlane_f32(m, 0), S = readlane_f32(s, 0);
    lse_merge(M, S, readlane_f32(m, 16), readlane_f32(s, 16), c);
    float M2 = readlane_f32(m, 32), S2 = readlane_f32(s, 32);
    lse_merge(M2, S2, readlane_f32(m, 48), readlane_f32(s, 48), c);
    lse_merge(M, S, M2, S2, c);
    m = M;
    s = S;
}

// Best kK keys of up to kPer*64 keys held kPer per lane (0 = empty).
// Returns, in lane r < kK, the r-th best key (0 if fewer exist); *count gets
// how many were found.  Each round finds the largest high word across the
// wave, then the largest low word among keys with that high word (keys are
// unique).
template <int kK, int kPer>
__device__ __forceinline__ uint64_t wave_select(uint64_t (&e)[kPer], int lane, uint32_t *count) {
    uint64_t mine = 0;
    uint32_t found = 0;
#pragma unroll 1
    for (int r = 0; r < kK; ++r) {
        uint64_t b = e[0];
#pragma unroll
        for (int i = 1; i < kPer; ++i) b = umax64(b, e[i]);
        const uint32_t bh = uint32_t(b >> 32);
        const uint32_t H = wave_max_u32(bh);
        if (H == 0) break;  // uniform: nothing left
        const uint32_t L = wave_max_u32(bh == H ? uint32_t(b) : 0u);
        const uint64_t win = (uint64_t(H) << 32) | L;
#pragma unroll
        for (int i = 0; i < kPer; ++i) e[i] = (e[i] == win) ? 0ull : e[i];
        if (lane == r) mine = win;
        ++found;
    }
    *count = found;
    return mine;
}

// Fewest slots for which a chunk's candidates are merged into the wave's
// list in bulk (gathered, then placed by rank) rather than one key at a
// time.  At 63 slots the list spans four rows of 16 lanes and a chunk still
// brings several keys once the seed has set the bound; at 31 the seed
// leaves so few that single insertions cost less (decode, 256 rows of
// 128256: 28.3 us with bulk merging, 27.5 without).
constexpr int kBulkMinK = 63;
// Fewest slots for which the seed waits (a barrier) for the chunks every
// wave holds at the start and ranks 4 maxima per lane instead of 1.
constexpr int kSeedAllMinK = 31;
// Gathered keys that a wave inserts one at a time rather than merging: a
// merge costs about as much as three or four single insertions.
constexpr uint32_t kBulkFewKeys = 3;
// Keys a wave gathers before it merges them.  Once the seed has set the
// bound a chunk brings a few keys, and a merge after every chunk cost more
// than the keys an earlier rise of the bound would have stopped; merging
// only when the 64 slots fill let the bound lag on long rows.  Same box at
// 63 slots, merging after every chunk / at 16 keys / at 64: ragged mix
// 27.9 / 25.9 / 25.2 us, decode 32.1 / 30.7 / 32.1 us, tie workload 596 /
// 596 / 600 us.
constexpr uint32_t kBulkMergeAt = 16;

__device__ __forceinline__ uint32_t lanes_below(uint64_t mask) {
    return __builtin_amdgcn_mbcnt_hi(uint32_t(mask >> 32), __builtin_amdgcn_mbcnt_lo(uint32_t(mask), 0u));
}

// The number of keys above `key` in a list of kK keys sorted in descending
// order (0 for empty slots), kK = 2^L - 1: a branchless binary search of L
// probes.
template <int kK>
__device__ __forceinline__ uint32_t count_above(const uint64_t *list, uint64_t key) {
    uint32_t pos = 0;
#pragma unroll
    for (uint32_t step = (uint32_t(kK) + 1) / 2; step > 0; step >>= 1)
        if (list[pos + step - 1] > key) pos += step;
    return pos;
}

// The number of keys above `key` in kN lists of kK keys each, sorted in
// descending order and stored one after another: the same binary search as
// count_above in every list, taken a probe at a time across the lists, so
// the kN reads of one probe go out together and the search costs
// log2(kK + 1) LDS round trips, not that many per group of lists.
template <int kK, int kN>
__device__ __forceinline__ uint32_t count_above_lists(const uint64_t *lists, uint64_t key) {
    uint32_t pos[kN];
#pragma unroll
    for (int w = 0; w < kN; ++w) pos[w] = 0;
#pragma unroll
    for (uint32_t step = (uint32_t(kK) + 1) / 2; step > 0; step >>= 1) {
        uint64_t v[kN];
#pragma unroll
        for (int w = 0; w < kN; ++w) v[w] = lists[w * kK + pos[w] + step - 1];
#pragma unroll
        for (int w = 0; w < kN; ++w)
            if (v[w] > key) pos[w] += step;
    }
    uint32_t n = 0;
#pragma unroll
    for (int w = 0; w < kN; ++w) n += pos[w];
    return n;
}

// ------------------------------------------------------------------ candidates
//
// Each wave keeps the K best keys it has seen (K = 2^levels - 1, 7 by
// default), sorted, one per lane in lanes 0..K-1 (0 = empty).  A wave filters
// its elements against a bound T: a key at or below T cannot be in the row's
// top K, because K real keys above it are known.  T is the larger of the
// wave's own K-th key and a workgroup-wide bound in LDS, which every wave
// raises (atomic max) whenever its own bound rises: any wave's K-th key bounds
// the whole row, since the K keys above it are real elements of the row.  A
// seed starts T off from the first chunks' lane maxima.
// For 31 or more slots the waves also publish one sorted position of their
// lists, whose minimum over the waves bounds the row more tightly.

// The smallest value a key above T can have (below the key of -inf, nothing
// is excluded): a float compare with it is a superset test for candidates,
// ties to be settled by the key compare.
__device__ __forceinline__ float threshold_value(uint64_t T) {
    return uint32_t(T >> 32) >= 0x007FFFFFu ? key_value(T) : -INFINITY;
}

// The smallest value strictly above T's value.  For a chunk whose ids all
// exceed T's id, an element beats T exactly when its value is above T's, so
// the float compare with this is exact there.
__device__ __forceinline__ float strict_value(uint64_t T) {
    const uint32_t hi = uint32_t(T >> 32);
    return hi >= 0x007FFFFFu ? key_value(uint64_t(hi + 1u) << 32) : -INFINITY;
}

// The larger of two logits.  Logits hold no NaN, so the IEEE maximum (which
// propagates NaN and orders -0 below +0, neither of which changes a max
// used as an exponent offset or as a superset test) serves; on gfx950 it is
// v_maximum3_f32, which needs no quieting of its inputs, where fmaxf costs
// a canonicalising max per loaded operand.
__device__ __forceinline__ float max_nan_free(float a, float b) { return __builtin_elementwise_maximum(a, b); }

__device__ __forceinline__ float group_max(const f32x4 &v) {
    return max_nan_free(max_nan_free(v.x, v.y), max_nan_free(v.z, v.w));
}

__device__ __forceinline__ float f4_get(const f32x4 &v, int q) {
    return q == 0 ? v.x : q == 1 ? v.y : q == 2 ? v.z : v.w;
}

// The high word of a value's order key: larger values map to larger words.
__device__ __forceinline__ uint32_t order_value(float v) { return uint32_t(order_key(v, kPadId) >> 32); }

// A bound from kN distinct real elements per lane, given as order values (0
// for none): if `need` of them are >= t (counting ties), no element below t
// can be in the top `need`, so the bound may be just under the smallest key
// of value t.  t is the need-th largest of the values cut to their top 16
// bits (sign, exponent and 7 mantissa bits: within 1/128 of it), found bit
// by bit from the top: a bit stays set when at least `need` values are at or
// above the prefix with it, 16 compare-and-count steps for any count.  A
// -inf t excludes nothing.
template <int kN>
__device__ __forceinline__ uint64_t bound_from_lane_values(const uint32_t (&u)[kN], uint32_t need) {
    uint32_t t = 0;
#pragma unroll
    for (int b = 31; b >= 16; --b) {
        const uint32_t trial = t | (1u << b);
        uint32_t n = 0;
#pragma unroll
        for (int i = 0; i < kN; ++i) n += uint32_t(__popcll(__ballot(u[i] >= trial)));
        if (n >= need) t = trial;
    }
    return t > 0 ? (uint64_t(t) << 32) - 1 : 0ull;  // low word 0: smallest key of value t
}

// Inserts the wave-uniform key k into the sorted list in lanes 0..kK-1: lane
// i takes k if k lands at position i, its upper neighbour's key if k lands
// above it (a one-lane shift), else keeps its own.  Other lanes stay 0.
template <int kK>
__device__ __forceinline__ uint64_t list_insert(uint64_t list, uint64_t k, int lane) {
    uint32_t ph, pl;
    if constexpr (kK <= 16) {
        // the list lies within the first row of 16 lanes: DPP row_shr:1
        constexpr int kDppShr1 = 0x111;
        ph = uint32_t(__builtin_amdgcn_update_dpp(-1, int(uint32_t(list >> 32)), kDppShr1, 0xF, 0xF, false));
        pl = uint32_t(__builtin_amdgcn_update_dpp(-1, int(uint32_t(list)), kDppShr1, 0xF, 0xF, false));
    } else {
        // across rows: a permute from lane - 1
        const int src = (lane > 0 ? lane - 1 : 0) * 4;
        ph = uint32_t(__builtin_amdgcn_ds_bpermute(src, int(uint32_t(list >> 32))));
        pl = uint32_t(__builtin_amdgcn_ds_bpermute(src, int(uint32_t(list))));
    }
    const uint64_t above = lane == 0 ? ~0ull : ((uint64_t(ph) << 32) | pl);
    const uint64_t next = k > list ? (k > above ? above : k) : list;
    return lane < kK ? next : 0ull;
}

// ------------------------------------------------------------------ row kernel

struct RowArgs {
    const float *src;          // logits the op reads: rows of row_len floats
    uint32_t row_len;          // V, or the width of a vocabulary shard
    uint32_t id_base;          // token id of a row's first element (a shard's first id)
    uint32_t split;            // segments per row
    uint32_t seg_len;          // elements per segment (multiple of 4)
    uint32_t out_rows;
    uint32_t records;          // 0: write the rows; 1: one record per (row, segment)
    uint64_t rec_row_stride;   // 8-byte words between two rows' records
    uint64_t rec_seg_stride;   // words between a row's segment records
    const RowDesc *desc;
    float *out_lp;             // rows: (R, kK + 1)
    uint32_t *out_id;          // rows: (R, kK + 1)
    uint64_t *rec;             // records of kK + 2 words (see below)
};

// A partial record, in 8-byte words: word 0 holds the segment's max and
// scaled sum (two floats), words 1..kK its best keys (descending, 0 past the
// ones it has), word kK + 1 the chosen token's logit (a float) and a flag
// set when the chosen token lies in the segment.

// log p = (x - M) / temperature - ln S for a row whose max is M and whose
// S = sum of e^((x - M) / temperature): the subtraction comes first, so a
// large common offset of the row costs no accuracy, and it is done in fp64,
// so logits at opposite ends of the fp32 range still give the finite value
// that the division by a large temperature brings back into range.  The
// division itself is in fp64 too: (x - M) is exact there, so the quotient
// carries no more than fp64 rounding, and the one rounding to fp32 at the
// end is the only one of size (a few lanes per row: the cost is nil).
__device__ __forceinline__ float logprob(float x, float M, float temp, float ln_s) {
    const double d = double(x) - double(M);
    // temperature 1 (a wave-uniform test) divides by nothing: d / 1 is d
    return float((temp == 1.0f ? d : d / double(temp)) - double(ln_s));
}

// One output row of kK + 1 columns: lanes 0..kK-1 the ranked slots, lane kK
// the chosen token.
// Sum over the wave, in a fixed order (every lane gets it).
__device__ __forceinline__ float wave_sum_f32(float v) {
    v += dpp_f32<kDppXor1>(v);
    v += dpp_f32<kDppXor2>(v);
    v += dpp_f32<kDppHalfMirror>(v);
    v += dpp_f32<kDppMirror>(v);
    return (readlane_f32(v, 0) + readlane_f32(v, 16)) + (readlane_f32(v, 32) + readlane_f32(v, 48));
}

__device__ __forceinline__ float wave_max_f32(float v) {
    v = max_nan_free(v, dpp_f32<kDppXor1>(v));
    v = max_nan_free(v, dpp_f32<kDppXor2>(v));
    v = max_nan_free(v, dpp_f32<kDppHalfMirror>(v));
    v = max_nan_free(v, dpp_f32<kDppMirror>(v));
    return max_nan_free(max_nan_free(readlane_f32(v, 0), readlane_f32(v, 16)),
                        max_nan_free(readlane_f32(v, 32), readlane_f32(v, 48)));
}

// The maximum and the sum over the first kN (4, 8 or 16) lanes, every lane
// of the first row of 16 taking part (lanes kN..15 must hold -inf, or 0 for
// the sum); the sum's order is fixed.
template <int kN>
__device__ __forceinline__ float first_lanes_max_f32(float v) {
    static_assert(kN == 4 || kN == 8 || kN == 16, "4, 8 or 16 lanes");
    v = max_nan_free(v, dpp_f32<kDppXor1>(v));
    v = max_nan_free(v, dpp_f32<kDppXor2>(v));
    if constexpr (kN >= 8) v = max_nan_free(v, dpp_f32<kDppHalfMirror>(v));
    if constexpr (kN >= 16) v = max_nan_free(v, dpp_f32<kDppMirror>(v));
    return readlane_f32(v, 0);
}
template <int kN>
__device__ __forceinline__ float first_lanes_sum_f32(float v) {
    static_assert(kN == 4 || kN == 8 || kN == 16, "4, 8 or 16 lanes");
    v += dpp_f32<kDppXor1>(v);
    v += dpp_f32<kDppXor2>(v);
    if constexpr (kN >= 8) v += dpp_f32<kDppHalfMirror>(v);
    if constexpr (kN >= 16) v += dpp_f32<kDppMirror>(v);
    return readlane_f32(v, 0);
}

// Writes an output row from the row's best keys (lane i < kK holds the
// (i+1)-th), its max M and scaled sum S.  top_word is the descriptor's third
// word: top_n, and in its high half the top-k front end's k.  With k > 0 the
// row's distribution is the softmax of the k kept logits alone (the TopK
// processor on logits, then Softmax, of the FlashInfer page): S becomes
// their sum, only kept tokens are listed, and a chosen token outside them
// gets -inf.
template <int kK>
__device__ __forceinline__ void write_row(float *out_lp, uint32_t *out_id, uint64_t o, int lane,
                                          uint64_t key, uint32_t top_word, float M, float S,
                                          float temp, float c, float x_chosen, uint32_t chosen) {
    constexpr uint64_t kC = uint64_t(kK) + 1;
    uint32_t listed = top_word & 0xFFFFu;
    const uint32_t keep = top_word >> 16;
    bool chosen_kept = true;
    if (keep != 0) {
        const bool kept = uint32_t(lane) < keep && key != 0;
        const float ms = (M == -INFINITY) ? 0.0f : M;
        S = wave_sum_f32(kept ? fast_exp2((key_value(key) - ms) * c) : 0.0f);
        chosen_kept = __ballot(kept && key_id(key) == chosen) != 0;
        if (keep < listed) listed = keep;
    }
    const float ln_s = logf(S);
    // lanes 0..kK-1 the ranked slots, lane kK the chosen token: one pass, so
    // the fp64 arithmetic runs once for all of them
    const bool ranked = lane < kK;
    const bool valid = ranked ? (uint32_t(lane) < listed && key != 0) : chosen_kept;
    const float x = ranked ? key_value(key) : x_chosen;
    const uint32_t id = ranked ? (valid ? key_id(key) : kPadId) : chosen;
    float lp = -INFINITY;
    if (valid) lp = logprob(x, M, temp, ln_s);
    if (lane <= kK) {
        out_lp[o * kC + lane] = lp;
        out_id[o * kC + lane] = id;
    }
}

// The whole descriptor of a workgroup's row in one 16-byte load, its fields
// made wave-uniform.
__device__ __forceinline__ RowDesc load_desc_uniform(const RowDesc *desc, uint32_t o) {
    const uint4 v = *reinterpret_cast<const uint4 *>(desc + o);
    return RowDesc{uint32_t(__builtin_amdgcn_readfirstlane(int(v.x))),
                   uint32_t(__builtin_amdgcn_readfirstlane(int(v.y))),
                   uint32_t(__builtin_amdgcn_readfirstlane(int(v.z))),
                   uint32_t(__builtin_amdgcn_readfirstlane(int(v.w)))};
}

// The descriptor of a workgroup's row as one 16-byte vector load (every lane
// loads the same 16 bytes; one request per wave).  Vector loads return in
// issue order, so a descriptor loaded ahead of the row's first chunks has
// arrived by the time those chunks have, and waiting for it never waits for
// anything else; a scalar load would share its counter with the LDS
// operations, and the first LDS wait would then stall on it.
__device__ __forceinline__ uint4 load_desc_vector(const RowDesc *desc, uint32_t o, uint32_t rows) {
    const __amdgpu_buffer_rsrc_t r =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<RowDesc *>(desc), 0, int(rows * uint32_t(sizeof(RowDesc))), kBufferWord3);
    return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, o * uint32_t(sizeof(RowDesc)), 0, 0));
}

__device__ __forceinline__ RowDesc desc_uniform(const uint4 v) {
    return RowDesc{uint32_t(__builtin_amdgcn_readfirstlane(int(v.x))),
                   uint32_t(__builtin_amdgcn_readfirstlane(int(v.y))),
                   uint32_t(__builtin_amdgcn_readfirstlane(int(v.z))),
                   uint32_t(__builtin_amdgcn_readfirstlane(int(v.w)))};
}

// Keys a row needs exactly: its top_n, or with the top-k front end its k
// (the kept keys all enter the renormalised sum; k >= the listed slots),
// within [1, kK].
template <int kK>
__device__ __forceinline__ uint32_t keys_needed(uint32_t top_word) {
    const uint32_t raw = (top_word >> 16) != 0 ? (top_word >> 16) : (top_word & 0xFFFFu);
    return raw < 1u ? 1u : (raw > uint32_t(kK) ? uint32_t(kK) : raw);
}

template <int kK>
__device__ __forceinline__ void write_padding(float *out_lp, uint32_t *out_id, uint64_t o, int lane) {
    constexpr uint64_t kC = uint64_t(kK) + 1;
    if (lane <= kK) {
        out_lp[o * kC + lane] = -INFINITY;
        out_id[o * kC + lane] = kPadId;
    }
}

// kDirect: output row o reads logits row o and no row is padding-only, so
// the row's address does not wait for its descriptor: its loads go out
// first, behind one vector load of the descriptor, whose fields are read
// when the first chunk has arrived.
// kK: ranked slots per row (2^levels - 1).
// kDyn: chunks past each wave's first kDepth are handed out one at a time as
// buffers free up (the waves of a workgroup then finish together), so which
// wave sums which chunk, and with it the fp32 rounding of the row's sum,
// depends on timing; without it the assignment is fixed and results are
// reproducible bit for bit.
template <int kK, int kWaves, int kDepth, bool kDirect, bool kDyn>
__global__ __launch_bounds__(kWaves * kWave) void row_kernel(RowArgs a) {
    constexpr int kThreads = kWaves * kWave;
    static_assert(kThreads >= kChunkF4, "one thread per float4 of the partial chunk");
    static_assert(kK >= 1 && kK < kWave, "one lane per column");
    // The seed's per-position maxima over the waves' first chunks, as order
    // values: with 31 or more slots 4 per lane (one per float4 group) once
    // every wave has added its own, else one per lane from whichever waves
    // have added theirs.
    constexpr bool kSeedAll = kK >= kSeedAllMinK;
    constexpr int kSeedN = kSeedAll ? kU : 1;
    __shared__ uint32_t s_lmax[kSeedN * kWave];
    __shared__ uint64_t s_keys[kWaves * kK];
    __shared__ uint64_t s_top[kK];
    __shared__ uint64_t s_T;
    __shared__ uint64_t s_pub[kWaves];
    __shared__ float2 s_lms[kWaves * kWave];   // every lane's (m, s)
    __shared__ float s_ms2[2];
    __shared__ uint32_t s_next;   // next chunk index to hand out (kDyn)
    constexpr bool kBulk = kK >= kBulkMinK;
    __shared__ uint64_t s_cand[kBulk ? kWaves * kWave : 1];   // per wave: gathered keys not yet merged
    __shared__ uint64_t s_new[kBulk ? kWaves * kK : 1];       // per wave: the merged list

    const int tid = int(threadIdx.x);
    const int lane = tid & (kWave - 1);
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: loop control stays scalar
    const uint32_t o = blockIdx.x / a.split;
    const uint32_t seg = blockIdx.x - o * a.split;
    constexpr int kPubJ = (kK + kWaves - 1) / kWaves - 1;        // published slot
    constexpr int kPubM = (kK + kPubJ) / (kPubJ + 1);           // waves needed
    constexpr bool kPubBound = kK >= 31 && kPubM >= kWaves;       // their minimum
    // The bound is the wave's need-th key (keys_needed): need real keys above
    // a key exclude it.  Slots past `need` are written as padding, so keys
    // there may be incomplete.  With direct rows the descriptor (and so
    // need, the temperature and the chosen token) is read after the first
    // chunk has arrived.
    uint4 dv{};
    RowDesc d{};
    if constexpr (kDirect) {
        dv = load_desc_vector(a.desc, o, a.out_rows);
    } else {
        d = load_desc_uniform(a.desc, o);
    }
    uint32_t need = keys_needed<kK>(d.top_n);

    if (!kDirect && d.top_n == 0) {  // padding-only row: no logits read (the merge kernel pads record rows)
        if (!a.records && wave == 0) write_padding<kK>(a.out_lp, a.out_id, o, lane);
        return;
    }

    const uint32_t V = a.row_len;
    const uint32_t gid = a.id_base;  // global id = gid + position in the row
    const float *row = a.src + uint64_t(kDirect ? o : d.src_row) * V;
    const uint64_t seg_start = uint64_t(seg) * a.seg_len;
    const uint32_t v0 = seg_start < V ? uint32_t(seg_start) : V;
    const uint32_t v1 = (uint64_t(v0) + a.seg_len < V) ? v0 + a.seg_len : V;

    // [v0, a0): < 4 elements before the first 16-byte boundary; [a0, a0 + 4 nf4):
    // float4s, nchunks full chunks of 1024 elements then a partial chunk;
    // then < 4 trailing elements
    uint32_t nh = (4u - uint32_t((reinterpret_cast<uintptr_t>(row + v0) >> 2) & 3u)) & 3u;
    if (nh > v1 - v0) nh = v1 - v0;
    const uint32_t a0 = v0 + nh;
    const uint32_t nf4 = (v1 - a0) >> 2;
    const uint32_t nchunks = nf4 / uint32_t(kChunkF4);
    const uint32_t ntr = (v1 - a0) & 3u;

    // the row's temperature; sums are of e^((x - m) / temperature) (with
    // direct rows both are set when the descriptor is read)
    float temp = kDirect ? 1.0f : __uint_as_float(d.temp_bits);
    float c = kDirect ? 0.0f : exp2_scale(temp);
    float m = -INFINITY, s = 0.0f;  // this lane's running max and sum of e^((x - m) / temperature)
    uint64_t list = 0;              // lane i < kK: the wave's (i+1)-th best key so far
    uint64_t T = 0;                 // wave-uniform bound (see above)
    uint32_t pending = 0;           // large K: keys in this wave's s_cand slots, not yet merged

    // The full chunks are read through a buffer resource whose range ends at
    // the last of them: a load past the end returns zeros without touching
    // memory.  So refills are unconditional, no buffer value ever merges two
    // paths, and the compiler keeps each buffer in place instead of copying
    // buffers at the loop's back edge (a copy would first wait for every load
    // in flight).  The partial chunk has a range of its own, so the refills
    // past the end never read it a second time.
    const StreamRange chunks = make_stream_range(row + a0, nchunks * uint32_t(kChunkF4 * 16));
    const StreamRange body = make_stream_range(row + a0, nf4 * 16u);
    auto load_chunk = [&](f32x4 (&x)[kU], uint32_t ch) __attribute__((always_inline)) {
        const uint32_t off = ch * uint32_t(kChunkF4 * 16) + uint32_t(lane) * 16u;
#pragma unroll
        for (int u = 0; u < kU; ++u) x[u] = stream_load(chunks, off + uint32_t(u * kWave * 16));
    };
    // Scheduling barriers keep the loads where they are: after the last use
    // of the buffer's old values (so the new ones can take the same
    // registers) and ahead of the wait for the next buffer (so that the other
    // loads stay in flight meanwhile).
    auto refill = [&](f32x4 (&x)[kU], uint32_t ch) __attribute__((always_inline)) {
        __builtin_amdgcn_sched_barrier(0);
        load_chunk(x, ch);
        __builtin_amdgcn_sched_barrier(0);
    };

    // the lane's chunk max: 16 values in 8 three-input maxima, a float4 at a
    // time as they arrive
    auto chunk_max = [&](const f32x4 (&x)[kU]) __attribute__((always_inline)) {
        float cm = max_nan_free(max_nan_free(x[0].x, x[0].y), max_nan_free(x[0].z, x[0].w));
#pragma unroll
        for (int u = 1; u < kU; ++u)
            cm = max_nan_free(max_nan_free(max_nan_free(cm, x[u].x), x[u].y), max_nan_free(x[u].z, x[u].w));
        return cm;
    };
    // the LSE update for a chunk whose lane max is cm
    auto lse_from = [&](const f32x4 (&x)[kU], float cm) __attribute__((always_inline)) {
        const float mn = fmaxf(m, cm);
        const float ms = (mn == -INFINITY) ? 0.0f : mn;
        float acc[kU];
#pragma unroll
        for (int u = 0; u < kU; ++u) {
            acc[u] = fast_exp2((x[u].x - ms) * c) + fast_exp2((x[u].y - ms) * c) +
                     (fast_exp2((x[u].z - ms) * c) + fast_exp2((x[u].w - ms) * c));
        }
        const float csum = (acc[0] + acc[1]) + (acc[2] + acc[3]);
        s = s * fast_exp2((m - ms) * c) + csum;
        m = mn;
    };
    auto lse_chunk = [&](const f32x4 (&x)[kU]) __attribute__((always_inline)) {
        const float cm = chunk_max(x);
        lse_from(x, cm);
        return cm;
    };

    // One column: a value and an id per lane, lanes passing tv_l tested
    // further (a lane that must not take part passes tv_l = +inf).  Keys above
    // T go into the list one at a time in lane order; T rises as it fills.
    auto column = [&](float v, uint32_t id, float tv_l) __attribute__((always_inline)) {
        const bool pass = v >= tv_l;
        if (__ballot(pass) == 0) return;
        const uint64_t key = order_key(v, id);
        uint64_t mask = __ballot(pass && key > T);
        while (mask != 0) {
            const int l = __builtin_ctzll(mask);
            list = list_insert<kK>(list, readlane_u64(key, l), lane);
            T = umax64(T, readlane_u64(list, int(need) - 1));
            mask = __ballot(pass && key > T) & ~((2ull << l) - 1ull);
        }
    };

    // A bound from every wave's (kPubJ+1)-th key: kPubM of them at or above x
    // mean kPubM * (kPubJ + 1) >= kK real keys at or above x (the waves'
    // shares are disjoint, and a published key only grows, so stale reads
    // are weaker, never wrong).  Tighter than the largest K-th key of one
    // wave; it pays only for large K.  Lane w < kWaves reads wave w's key,
    // and a DPP minimum over those lanes gives the bound (8 LDS reads in a
    // row cost about as much as one insertion).
    auto publish_bound = [&]() __attribute__((always_inline)) {
        if constexpr (kPubBound) {
            static_assert(kPubM == kWaves, "every wave's key is needed");
            const uint64_t mine = readlane_u64(list, kPubJ);
            if (lane == 0) __hip_atomic_store(&s_pub[wave], mine, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
            uint64_t v = ~0ull;
            if (lane < kWaves) v = lane == wave ? mine : lds_load_relaxed(&s_pub[lane]);
            T = umax64(T, first_lanes_min_u64<kWaves>(v));
        }
    };

    // Large K: merges the n keys a wave has gathered in its s_cand slots (keys
    // above T, distinct, unsorted) into its sorted list.  A list key's new
    // position is its old one plus the gathered keys above it, counted with
    // broadcast reads; a gathered key's is the gathered keys above it plus
    // the list keys above it, found by binary search.  The keys are distinct,
    // so the positions are too; the first kK are kept, and T rises to the
    // need-th, then the published bound is refreshed.  About one insertion's
    // cost, whatever n (<= 64).
    auto bulk_merge = [&](uint32_t n) __attribute__((always_inline)) {
        uint64_t *cand = s_cand + wave * kWave;
        uint64_t *sl = s_keys + wave * kK;   // this wave's slots, free until the end
        uint64_t *nl = s_new + wave * kK;
        if (lane < kK) {
            sl[lane] = list;
            nl[lane] = 0ull;
        }
        lds_release();
        lds_acquire();
        const uint64_t mine = uint32_t(lane) < n ? cand[lane] : 0ull;
        uint32_t above_l = 0, above_c = 0;
#pragma unroll 4
        for (uint32_t k = 0; k < n; ++k) {
            const uint64_t b = cand[k];   // a broadcast read
            above_l += b > list ? 1u : 0u;
            above_c += b > mine ? 1u : 0u;
        }
        if (lane < kK && list != 0) {
            const uint32_t r = uint32_t(lane) + above_l;
            if (r < uint32_t(kK)) nl[r] = list;
        }
        if (mine != 0) {
            const uint32_t r = above_c + count_above<kK>(sl, mine);
            if (r < uint32_t(kK)) nl[r] = mine;
        }
        lds_release();
        lds_acquire();
        list = lane < kK ? nl[lane] : 0ull;
        T = umax64(T, readlane_u64(list, int(need) - 1));
        publish_bound();
    };

    // The filter value for chunk ch against the bound as it stands.
    auto chunk_tv = [&](uint32_t ch) __attribute__((always_inline)) {
        const uint32_t first = gid + a0 + ch * uint32_t(kChunkF4 * 4);
        return key_id(T) < first ? strict_value(T) : threshold_value(T);
    };

    // Top-k part for one chunk whose lane maxima are cm: a ballot of the lane
    // maxima against tv passes most chunks by; else one ballot per float4
    // group and per column finds the columns holding candidates, which then
    // go through a single copy of the column code (uniform register indexing).
    auto topk_chunk = [&](const f32x4 (&x)[kU], uint32_t ch, float cm) __attribute__((always_inline)) {
        const float tv = chunk_tv(ch);
        if (__ballot(cm >= tv) == 0) return;
        const uint64_t T0 = T;
        static_assert(kU == 4, "16 columns per chunk");
        uint32_t cols = 0;
#pragma unroll
        for (int u = 0; u < kU; ++u) {
            const float gm = group_max(x[u]);
            if (__ballot(gm >= tv) == 0) continue;
#pragma unroll
            for (int q = 0; q < 4; ++q)
                cols |= (__ballot(f4_get(x[u], q) >= tv) != 0 ? 1u : 0u) << (4 * u + q);
        }
        const f32x16 xv = __builtin_shufflevector(__builtin_shufflevector(x[0], x[1], 0, 1, 2, 3, 4, 5, 6, 7),
                                                  __builtin_shufflevector(x[2], x[3], 0, 1, 2, 3, 4, 5, 6, 7),
                                                  0, 1, 2, 3, 4, 5, 6, 7, 8, 9, 10, 11, 12, 13, 14, 15);
        const uint32_t lane_id = gid + a0 + ch * uint32_t(kChunkF4 * 4) + 4u * uint32_t(lane);
        if constexpr (kBulk) {
            // gather the keys above T column by column into this wave's
            // s_cand slots (ballot and lane prefix), merging first whenever a
            // column would overflow the 64 slots; the slots are merged once
            // they hold kBulkMergeAt keys and after the wave's last chunk,
            // not after every chunk
            uint64_t *cand = s_cand + wave * kWave;
            while (cols != 0) {
                const uint32_t j = uint32_t(__builtin_ctz(cols));
                cols &= cols - 1;
                const float v = xv[j];
                const bool pass = v >= tv;
                const uint64_t key = order_key(v, lane_id + 4u * uint32_t(kWave) * (j >> 2) + (j & 3u));
                uint64_t mask = __ballot(pass && key > T);
                if (mask == 0) continue;
                if (pending + uint32_t(__popcll(mask)) > uint32_t(kWave)) {
                    bulk_merge(pending);
                    pending = 0;
                    mask = __ballot(pass && key > T);
                    if (mask == 0) continue;
                }
                if (pass && key > T) cand[pending + lanes_below(mask)] = key;
                pending += uint32_t(__popcll(mask));
            }
            if (pending >= kBulkMergeAt) {
                bulk_merge(pending);
                pending = 0;
            }
        } else {
            while (cols != 0) {
                const uint32_t j = uint32_t(__builtin_ctz(cols));
                cols &= cols - 1;
                column(xv[j], lane_id + 4u * uint32_t(kWave) * (j >> 2) + (j & 3u), tv);
            }
            publish_bound();
        }
        if (T != T0 && lane == 0) __hip_atomic_fetch_max(&s_T, T, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
    };

    f32x4 xb[kDepth][kU];
    uint32_t ch = uint32_t(wave);
#pragma unroll
    for (int dd = 0; dd < kDepth; ++dd) refill(xb[dd], ch + uint32_t(dd * kWaves));
    // The partial chunk (one float4 per thread), the head and trailing
    // elements (one per thread) and the chosen token's logit are loaded now,
    // so that their latency hides under the stream.
    const uint32_t rest4 = nchunks * uint32_t(kChunkF4) + uint32_t(tid);
    const bool rest4_ok = rest4 < nf4;
    const f32x4 xr4 = stream_load(body, rest4 * 16u);
    const bool e1_ok = uint32_t(tid) < nh + ntr;
    const uint32_t e1 = uint32_t(tid) < nh ? v0 + uint32_t(tid) : a0 + 4u * nf4 + (uint32_t(tid) - nh);
    const float xr1 = row[e1_ok ? e1 : 0u];
    // the chosen token's logit, from the segment that holds it (with direct
    // rows, once the descriptor is read, below)
    bool owns_chosen = false;
    float x_chosen = 0.0f;
    auto load_chosen = [&]() __attribute__((always_inline)) {
        const uint32_t chosen_local = d.chosen - gid;
        owns_chosen = d.chosen >= gid && chosen_local >= v0 && chosen_local < v1;
        x_chosen = row[(owns_chosen && lane == kK) ? chosen_local : 0u];
    };
    if constexpr (!kDirect) load_chosen();
    // LDS set-up (before any data can have arrived, so the barrier costs only
    // the spread of the waves' start)
    if (tid < kSeedN * kWave) s_lmax[tid] = 0u;
    if (tid < kWaves) s_pub[tid] = 0;
    if (tid == 0) {
        s_T = 0;
        s_next = uint32_t(kDepth * kWaves);
    }
    __syncthreads();

    {
        // First chunk.  With direct rows it is copied aside and its buffer
        // refilled at once, so that loads stay in flight while the wave
        // computes the seed and ranks the chunk's candidates (decode, 256
        // rows of 128256: 25.4 -> 25.0 us).  Rows found through their
        // descriptors refill after the chunk, as in the loop (the early
        // refill cost 1.3-1.5 us on 520 rows of 32000, one chunk deep).
        // The seed: distinct elements of the row bound it (the need-th
        // largest of any of them is at most the row's need-th), here the
        // per-position maxima of the waves' first chunks (see below).
        constexpr uint32_t kAhead = uint32_t(kDepth * kWaves);
        // With kDyn each wave takes its next chunk index from an LDS counter
        // one step ahead of the refill that needs it, so the atomic's
        // latency hides under a chunk.  cb[b] is the chunk buffer b holds.
        uint32_t cb[kDepth];
#pragma unroll
        for (int dd = 0; dd < kDepth; ++dd) cb[dd] = uint32_t(wave + dd * kWaves);
        auto grab = [&]() __attribute__((always_inline)) {
            uint32_t v = 0;
            if (kDyn && lane == 0)
                v = __hip_atomic_fetch_add(&s_next, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
            return v;   // lane 0's value, read with readfirstlane when used
        };
        uint32_t gv = grab();
        // refills buffer b with the next chunk: the grabbed one, or the one
        // kAhead past what it held
        auto refill_next = [&](f32x4 (&x)[kU], uint32_t &held) __attribute__((always_inline)) {
            held = kDyn ? uint32_t(__builtin_amdgcn_readfirstlane(int(gv))) : held + kAhead;
            refill(x, held);
            if constexpr (kDyn) gv = grab();
        };
        f32x4 x0[kU];
        if constexpr (kDirect) {
#pragma unroll
            for (int u = 0; u < kU; ++u) x0[u] = xb[0][u];
            refill_next(xb[0], cb[0]);
            d = desc_uniform(dv);
            need = keys_needed<kK>(d.top_n);
            temp = __uint_as_float(d.temp_bits);
            c = exp2_scale(temp);
            load_chosen();
        }
        f32x4 (&first)[kU] = kDirect ? x0 : xb[0];
        float cm0 = -INFINITY;
        if (ch < nchunks) cm0 = lse_chunk(first);
        if constexpr (kSeedAll) {
            // per (float4 group, lane) the largest of the waves' group
            // maxima over all the chunks they hold (kDepth each): 256
            // distinct elements, each the largest of 4 * kWaves * kDepth
            // (two deep, levels 6: ragged mix 30.9 -> 27.9 us, decode 36.5
            // -> 34.4 us against the first chunk alone)
            uint32_t ux[kU];
#pragma unroll
            for (int u = 0; u < kU; ++u) {
                ux[u] = ch < nchunks ? order_value(group_max(first[u])) : 0u;
#pragma unroll
                for (int dd = 1; dd < kDepth; ++dd)
                    if (cb[dd] < nchunks) ux[u] = max(ux[u], order_value(group_max(xb[dd][u])));
                __hip_atomic_fetch_max(&s_lmax[u * kWave + lane], ux[u], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
            }
            __syncthreads();
#pragma unroll
            for (int u = 0; u < kU; ++u) ux[u] = s_lmax[u * kWave + lane];
            T = bound_from_lane_values<kU>(ux, need);
        } else {
            // per lane the largest chunk maximum of the waves that have added
            // theirs (this one's at least); a relaxed atomic, since other
            // waves add theirs with no barrier in between
            const uint32_t u0 = order_value(cm0);
            const uint32_t prev = __hip_atomic_fetch_max(&s_lmax[lane], u0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
            const uint32_t ux[1] = {prev > u0 ? prev : u0};
            T = bound_from_lane_values<1>(ux, need);
        }
        if (lane == 0 && T != 0) __hip_atomic_fetch_max(&s_T, T, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
        if (ch < nchunks) topk_chunk(first, ch, cm0);
        if constexpr (!kDirect) refill_next(xb[0], cb[0]);
        // the partial chunk and the single elements, from the registers they
        // were loaded into at the start: handled now, so that no wave has
        // them left to do after its last chunk
        {
            const f32x4 x4 = rest4_ok ? xr4 : f32x4{-INFINITY, -INFINITY, -INFINITY, -INFINITY};
            const float x1 = e1_ok ? xr1 : -INFINITY;
            const float cm = fmaxf(fmaxf(fmaxf(x4.x, x4.y), fmaxf(x4.z, x4.w)), x1);
            const float mn = fmaxf(m, cm);
            const float ms = (mn == -INFINITY) ? 0.0f : mn;
            const float add = (fast_exp2((x4.x - ms) * c) + fast_exp2((x4.y - ms) * c)) +
                              (fast_exp2((x4.z - ms) * c) + fast_exp2((x4.w - ms) * c)) +
                              fast_exp2((x1 - ms) * c);
            s = s * fast_exp2((m - ms) * c) + add;
            m = mn;
            T = umax64(T, uniform64(lds_load_relaxed(&s_T)));
            const float tv = threshold_value(T);
            if (__ballot(cm >= tv) != 0) {
                const uint32_t id4 = gid + a0 + 4u * rest4;
                const float tv4 = rest4_ok ? tv : INFINITY;
#pragma unroll
                for (int q = 0; q < 4; ++q) column(f4_get(x4, q), id4 + uint32_t(q), tv4);
                column(x1, gid + e1, e1_ok ? tv : INFINITY);
            }
        }
        // The remaining chunks of this wave go in whole rounds of kDepth steps
        // (buffer d % kDepth on the d-th step of a round).  Buffers are
        // processed in the order they were filled, so the chunk indices they
        // hold increase in that order: once the next one is past the end,
        // every later one is too, and the wave is done; within the last
        // round, steps past the end skip their chunk and their refill reads
        // nothing.  The loop has one exit, at its bottom, and no buffer is
        // read after it: an exit from the middle, or a use after the loop,
        // would add paths on which buffers are copied between registers or
        // every wait for loads in flight must be stricter.  The shared bound
        // is read before each chunk's arithmetic, so that its latency hides
        // there.
        if constexpr (kDepth == 1 && kK >= 31 && kWaves == 16) {
            // One chunk in flight per wave, in two buffers taken in turn: once
            // a chunk has arrived (its lane maxima are the first use) the
            // next chunk goes into the other buffer, whose chunk is done, and
            // only then does the arithmetic start, so the load is in flight
            // while the wave computes instead of after it.  It pays where a
            // chunk's work is long and a CU holds one workgroup: 31 and 63
            // slots at 16 waves (decode, 256 rows of 128256: levels 5 26.92
            // -> 26.51 us, levels 6 29.99 -> 29.59 us).  With 7 slots, or
            // several workgroups per CU, the extra bytes in flight cost more
            // than the overlap gains (decode at levels 3 22.78 -> 23.18 us,
            // 520 rows of 32000 at 8 waves 15.63 -> 17.39 us).
            f32x4 yb[kU];
            uint32_t cy = 0;
            auto refill_after = [&](f32x4 (&x)[kU], uint32_t &held, uint32_t prev) __attribute__((always_inline)) {
                held = kDyn ? uint32_t(__builtin_amdgcn_readfirstlane(int(gv))) : prev + uint32_t(kWaves);
                // the chunk being worked on has arrived: the only vector
                // loads in flight are its own (vmcnt(0); expcnt and lgkmcnt
                // left at their maxima, so nothing else is waited for)
                __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
                refill(x, held);
                if constexpr (kDyn) gv = grab();
            };
            while (cb[0] < nchunks) {
                {
                    const uint64_t shared = lds_load_relaxed(&s_T);
                    const float cm = chunk_max(xb[0]);
                    refill_after(yb, cy, cb[0]);
                    lse_from(xb[0], cm);
                    T = umax64(T, uniform64(shared));
                    topk_chunk(xb[0], cb[0], cm);
                }
                if (cy < nchunks) {
                    const uint64_t shared = lds_load_relaxed(&s_T);
                    const float cm = chunk_max(yb);
                    refill_after(xb[0], cb[0], cy);
                    lse_from(yb, cm);
                    T = umax64(T, uniform64(shared));
                    topk_chunk(yb, cy, cm);
                } else {
                    cb[0] = cy;   // past the end: every later index is too
                }
            }
        } else {
            while (cb[1 % kDepth] < nchunks) {
#pragma unroll
                for (int dd = 1; dd <= kDepth; ++dd) {
                    if (cb[dd % kDepth] < nchunks) {
                        const uint64_t shared = lds_load_relaxed(&s_T);
                        const float cm = lse_chunk(xb[dd % kDepth]);
                        T = umax64(T, uniform64(shared));
                        topk_chunk(xb[dd % kDepth], cb[dd % kDepth], cm);
                    }
                    refill_next(xb[dd % kDepth], cb[dd % kDepth]);
                }
            }
        }
    }

    if constexpr (kBulk) {
        // the keys still pending: merged, or a few inserted one at a time
        if (pending > kBulkFewKeys) {
            bulk_merge(pending);
        } else if (pending != 0) {
            lds_release();
            lds_acquire();
            const uint64_t *cand = s_cand + wave * kWave;
            for (uint32_t k = 0; k < pending; ++k) {
                const uint64_t key = uniform64(cand[k]);
                if (key > T) {
                    list = list_insert<kK>(list, key, lane);
                    T = umax64(T, readlane_u64(list, int(need) - 1));
                }
            }
        }
    }

    // per wave: its list and (m, s) across lanes into LDS; then every wave
    // ranks its share of the waves' kN (<= threads) keys, one per thread: a
    // key's rank is the number of keys above it in all the lists together
    // (in its own list, its position; the keys are distinct), each list
    // binary-searched in log2(kK + 1) probes, and the best kK go to their
    // rank.  Wave 0 then writes the row (or the segment's record).  The
    // last wave to arrive used to rank them all alone: kPer rounds of
    // searches (6.5 us at 63 slots), or at 7 slots counting or kK wave-wide
    // maxima; with every wave ranking, decode at 7 slots went 24.5 -> 23.7
    // us and the 4-row batch (16 waves) 9.0 -> 8.5 us, same box.
    //
    // The workgroup's (M, S) comes from plain reductions instead of pairwise
    // (m, s) merges (two exponentials each): before the first barrier every
    // lane stores its (m, s), and between the barriers the last wave takes
    // the maximum M of them all and the sum of every s scaled to M (one
    // exponential per stored pair), while the other waves rank.  Between the barriers only the ranking is
    // left (with the one-pass epilogue of write_row: 520 rows of 32000 15.62
    // -> 15.37 us, decode 22.84 -> 22.74 us, same box).
    if (lane < kK) s_keys[wave * kK + lane] = list;
    s_lms[wave * kWave + lane] = make_float2(m, s);
    constexpr int kN = kWaves * kK;
    static_assert(kN <= kThreads, "one key per thread");
    if (wave == 0 && lane < kK) s_top[lane] = 0ull;
    __syncthreads();
    // The last wave (idle in the ranking at up to 15 slots) reduces the
    // lanes' pairs while the others rank, so that neither the last wave to
    // finish its stream nor wave 0 after the second barrier spends time on
    // them (same box: decode 22.64 -> 22.53 us with the waves' own
    // reductions still before the barrier, 22.55 -> 22.37 us without them;
    // the 4-row batch 8.13 -> 8.01 -> 7.61 us).
    if (wave == kWaves - 1) {
        float2 v[kWaves];
#pragma unroll
        for (int w = 0; w < kWaves; ++w) v[w] = s_lms[w * kWave + lane];
        float ml = v[0].x;
#pragma unroll
        for (int w = 1; w < kWaves; ++w) ml = fmaxf(ml, v[w].x);
        const float M = wave_max_f32(ml);
        const float Ms = (M == -INFINITY) ? 0.0f : M;
        float sl = 0.0f;
#pragma unroll
        for (int w = 0; w < kWaves; ++w) sl += v[w].y * fast_exp2((v[w].x - Ms) * c);   // s = 0 where m = -inf
        const float S = wave_sum_f32(sl);
        if (lane == 0) {
            s_ms2[0] = M;
            s_ms2[1] = S;
        }
    }
    if (tid < kN) {
        const uint64_t key = s_keys[tid];
        if (key != 0) {
            uint32_t rank = 0;
            if constexpr (kK <= 15 && kWaves >= 8) {
                // all lists a probe at a time (decode, 256 rows of 128256:
                // 23.03 -> 22.91 us; 520 rows of 32000: 15.75 -> 15.71 us)
                rank = count_above_lists<kK, kWaves>(s_keys, key);
            } else {
                // longer searches, or four lists: list by list, which the
                // compiler already overlaps four at a time (the interleaved
                // form was 0.2-0.7 % slower at 31 and 63 slots)
#pragma unroll
                for (int w = 0; w < kWaves; ++w) rank += count_above<kK>(s_keys + w * kK, key);
            }
            if (rank < uint32_t(kK)) s_top[rank] = key;
        }
    }
    __syncthreads();
    if (wave != 0) return;
    const uint64_t top = lane < kK ? s_top[lane] : 0ull;
    const float M = s_ms2[0];
    const float S = s_ms2[1];

    if (!a.records) {
        write_row<kK>(a.out_lp, a.out_id, o, lane, top, d.top_n, M, S, temp, c, x_chosen, d.chosen);
    } else {
        uint64_t *rec = a.rec + uint64_t(o) * a.rec_row_stride + uint64_t(seg) * a.rec_seg_stride;
        if (lane == 0) {
            reinterpret_cast<float *>(rec)[0] = M;
            reinterpret_cast<float *>(rec)[1] = S;
        }
        if (lane < kK) rec[1 + lane] = top;
        if (lane == kK) {
            reinterpret_cast<float *>(rec + kK + 1)[0] = owns_chosen ? x_chosen : 0.0f;
            reinterpret_cast<uint32_t *>(rec + kK + 1)[1] = owns_chosen ? 1u : 0u;
        }
    }
}

// ------------------------------------------------------------------ merge kernel

struct MergeArgs {
    uint32_t nseg;             // records per row (segments, or vocabulary shards)
    uint32_t out_rows;
    uint64_t rec_row_stride;   // 8-byte words between two rows' records
    uint64_t rec_seg_stride;   // words between a row's records
    const RowDesc *desc;
    const uint64_t *rec;
    float *out_lp;
    uint32_t *out_id;
};

// Merges each row's records, one wave per output row: the (max, sum) pairs
// in record order, the best kK of all their keys, the chosen token's logit
// from the record that holds it (NaN if none does); then writes the row.
// nseg * kK <= kMaxMergeKeys, so kPer keys per lane hold them.
template <int kK>
__global__ __launch_bounds__(256) void merge_kernel(MergeArgs a) {
    constexpr int kPer = int((kMaxMergeKeys + kWave - 1) / kWave) < (int(kMaxSplit) * kK + kWave - 1) / kWave
                             ? int((kMaxMergeKeys + kWave - 1) / kWave)
                             : (int(kMaxSplit) * kK + kWave - 1) / kWave;
    const int lane = int(threadIdx.x) & (kWave - 1);
    const uint32_t o = blockIdx.x * 4u + (threadIdx.x >> 6);
    if (o >= a.out_rows) return;
    const RowDesc d = a.desc[o];
    if (d.top_n == 0) {
        write_padding<kK>(a.out_lp, a.out_id, o, lane);
        return;
    }
    const uint64_t *recs = a.rec + uint64_t(o) * a.rec_row_stride;
    float m = -INFINITY, s = 0.0f, xc = 0.0f;
    bool owner = false;
    if (uint32_t(lane) < a.nseg) {
        const uint64_t *r = recs + uint64_t(lane) * a.rec_seg_stride;
        const float *ms = reinterpret_cast<const float *>(r);
        m = ms[0];
        s = ms[1];
        xc = reinterpret_cast<const float *>(r + kK + 1)[0];
        owner = reinterpret_cast<const uint32_t *>(r + kK + 1)[1] != 0;
    }
    const uint64_t own = __ballot(owner);
    const float x_chosen = own != 0 ? readlane_f32(xc, __builtin_ctzll(own)) : __uint_as_float(0x7FC00000u);
    const float temp = __uint_as_float(d.temp_bits);
    const float c = exp2_scale(temp);
    wave_lse(m, s, c);
    const uint32_t nkeys = a.nseg * uint32_t(kK);
    // this wave's LDS: the records' keys (record r's slot p at r * kK + p)
    // and the kK best, placed by rank
    constexpr int kMaxKeys = int(kMaxMergeKeys) < int(kMaxSplit) * kK ? int(kMaxMergeKeys) : int(kMaxSplit) * kK;
    // from 7 slots up every key count is ranked by binary search over the
    // records (each record's keys are sorted), so the keys are staged in LDS
    constexpr bool kSearch = kK >= 7;
    constexpr int kSlots = kSearch && kMaxKeys > kWave ? kMaxKeys : kWave;
    __shared__ uint64_t s_k[4][kSlots];
    __shared__ uint64_t s_t[4][kWave];
    const int w = int(threadIdx.x >> 6);
    uint64_t top;
    if constexpr (kSearch) {
        // every record's keys are sorted, so a key's rank is the number of
        // keys above it summed over the records, each a binary search of
        // log2(kK + 1) probes in LDS; the best kK go to their rank
        for (uint32_t idx = uint32_t(lane); idx < nkeys; idx += kWave)
            s_k[w][idx] = recs[uint64_t(idx / kK) * a.rec_seg_stride + 1 + idx % kK];
        if (lane < kK) s_t[w][lane] = 0ull;
        lds_release();
        lds_acquire();
        for (uint32_t idx = uint32_t(lane); idx < nkeys; idx += kWave) {
            const uint64_t key = s_k[w][idx];
            if (key == 0) continue;
            uint32_t rank = 0;
            for (uint32_t r = 0; r < a.nseg; ++r) rank += count_above<kK>(&s_k[w][r * kK], key);
            if (rank < uint32_t(kK)) s_t[w][rank] = key;
        }
        lds_release();
        lds_acquire();
        top = lane < kK ? s_t[w][lane] : 0ull;
    } else if (nkeys <= uint32_t(kWave)) {
        // at most one key per lane: each key's rank is the number of keys
        // above it (keys of different records are distinct; empty slots are
        // 0 and never placed), counted with broadcast LDS reads from this
        // wave's own slots; the best kK go to their rank.  The fences keep
        // the compiler from forwarding a lane's own store to its read-back.
        const uint64_t mine = uint32_t(lane) < nkeys
                                  ? recs[uint64_t(uint32_t(lane) / kK) * a.rec_seg_stride + 1 + uint32_t(lane) % kK]
                                  : 0ull;
        s_k[w][lane] = mine;
        if (lane < kK) s_t[w][lane] = 0ull;
        lds_release();
        lds_acquire();
        uint32_t rank = 0;
#pragma unroll 8
        for (uint32_t j = 0; j < nkeys; ++j) rank += s_k[w][j] > mine ? 1u : 0u;
        lds_release();
        if (mine != 0 && rank < uint32_t(kK)) s_t[w][rank] = mine;
        lds_release();
        lds_acquire();
        top = lane < kK ? s_t[w][lane] : 0ull;
    } else {
        uint64_t e[kPer];
#pragma unroll
        for (int i = 0; i < kPer; ++i) {
            const uint32_t idx = uint32_t(lane + kWave * i);
            e[i] = idx < nkeys ? recs[uint64_t(idx / kK) * a.rec_seg_stride + 1 + idx % kK] : 0ull;
        }
        uint32_t found;
        top = wave_select<kK, kPer>(e, lane, &found);
    }
    write_row<kK>(a.out_lp, a.out_id, o, lane, top, d.top_n, m, s, temp, c, x_chosen, d.chosen);
}

// Plans that read no row (every top_n is 0): all R * columns entries padding.
__global__ __launch_bounds__(256) void pad_kernel(float *out_lp, uint32_t *out_id, uint64_t n) {
    for (uint64_t i = uint64_t(blockIdx.x) * 256u + threadIdx.x; i < n; i += uint64_t(gridDim.x) * 256u) {
        out_lp[i] = -INFINITY;
        out_id[i] = kPadId;
    }
}

// Descriptors carried in the launch's own arguments, copied into device
// memory: the runtime copies kernel arguments when the launch is enqueued,
// so the host array they came from is free again at once, with no pinned
// memory and no wait.  248 descriptors and the header make 3984 bytes of
// arguments, inside the 4 KB that kernel arguments may take; the kernel
// reads them from the argument segment with one 16-byte load per thread.
constexpr uint32_t kUploadRows = 248;

struct DescUpload {
    RowDesc d[kUploadRows];
    RowDesc *dst;              // the first of `count` descriptors to write
    uint32_t count;            // 1..kUploadRows
    uint32_t pad;
};
static_assert(sizeof(DescUpload) <= 4096, "kernel arguments are limited to 4 KB");

__global__ __launch_bounds__(256) void desc_upload_kernel(const DescUpload u) {
    const uint32_t t = threadIdx.x;
    if (t < u.count) u.dst[t] = u.d[t];
}

// ------------------------------------------------------------------ streaming-read probe

// One workgroup of 8 waves per row of row_len floats (16-byte aligned rows),
// each lane reading 4 nontemporal 16-byte loads per step -- the row-shaped
// plain read that sustains the most bandwidth on these shapes -- and writing
// the row's sum (so nothing is optimised away).
__global__ __launch_bounds__(512) void stream_read_kernel(const float *x, uint32_t row_len,
                                                         float *partial) {
    __shared__ float red[8];
    constexpr uint32_t kThreads = 512;
    const f32x4 *row = reinterpret_cast<const f32x4 *>(x + uint64_t(blockIdx.x) * row_len);
    const uint32_t n4 = row_len / 4;
    float acc = 0.0f;
    uint32_t i = threadIdx.x;
    for (; i + 3 * kThreads < n4; i += 4 * kThreads) {
        f32x4 v[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) v[u] = __builtin_nontemporal_load(row + i + u * kThreads);
#pragma unroll
        for (int u = 0; u < 4; ++u) acc += (v[u].x + v[u].y) + (v[u].z + v[u].w);
    }
    for (; i < n4; i += kThreads) {
        const f32x4 v = row[i];
        acc += (v.x + v.y) + (v.z + v.w);
    }
    if (threadIdx.x < row_len - n4 * 4) acc += x[uint64_t(blockIdx.x) * row_len + n4 * 4 + threadIdx.x];
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) acc += __shfl_xor(acc, o);
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = acc;
    __syncthreads();
    if (threadIdx.x == 0) {
        float t = 0.0f;
        for (int k = 0; k < 8; ++k) t += red[k];
        partial[blockIdx.x] = t;
    }
}

// The same plain read in other shapes, for a sweep of what the memory system
// gives this row shape: `segs` workgroups of kThreads per row, each reading
// one contiguous share of the row's float4s with kLoads nontemporal 16-byte
// loads in flight per thread, and writing its share's sum to
// partial[row * segs + seg].  row_len is a multiple of 4.
template <int kThreads, int kLoads>
__global__ __launch_bounds__(kThreads) void stream_read_shape_kernel(const float *x, uint32_t row_len,
                                                                     uint32_t segs, float *partial) {
    __shared__ float red[kThreads / 64];
    const uint32_t row = blockIdx.x / segs;
    const uint32_t seg = blockIdx.x - row * segs;
    const uint32_t n4 = row_len / 4;
    const uint32_t per = (n4 + segs - 1) / segs;
    const uint32_t b = seg * per < n4 ? seg * per : n4;
    const uint32_t e = b + per < n4 ? b + per : n4;
    const f32x4 *p = reinterpret_cast<const f32x4 *>(x + uint64_t(row) * row_len);
    float acc = 0.0f;
    uint32_t i = b + threadIdx.x;
    for (; i + uint32_t((kLoads - 1) * kThreads) < e; i += uint32_t(kLoads * kThreads)) {
        f32x4 v[kLoads];
#pragma unroll
        for (int u = 0; u < kLoads; ++u) v[u] = __builtin_nontemporal_load(p + i + u * kThreads);
#pragma unroll
        for (int u = 0; u < kLoads; ++u) acc += (v[u].x + v[u].y) + (v[u].z + v[u].w);
    }
    for (; i < e; i += kThreads) {
        const f32x4 v = __builtin_nontemporal_load(p + i);
        acc += (v.x + v.y) + (v.z + v.w);
    }
    acc = wave_sum_f32(acc);
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = acc;
    __syncthreads();
    if (threadIdx.x == 0) {
        float t = 0.0f;
        for (int k = 0; k < kThreads / 64; ++k) t += red[k];
        partial[blockIdx.x] = t;
    }
}

}  // namespace dev

// ------------------------------------------------------------------ host glue

static thread_local int g_last_hip_error = 0;

#define LP_HIP_TRY(expr)                          \
    do {                                          \
        const hipError_t e_ = (expr);             \
        if (e_ != hipSuccess) {                   \
            ::lp::g_last_hip_error = int(e_);     \
            return LP_ERR_HIP;                    \
        }                                         \
    } while (0)

// Pinned host staging for descriptor uploads, shared by every plan of the
// process: a slot belongs to one device and is reused once the event recorded
// after its last use has completed, so planning, staging and destroying a
// plan neither allocate pinned memory nor wait in the steady state.  Slots are
// never freed before the process ends (the pool only grows to the number of
// uploads in flight at once).
struct StagingSlot {
    void *host = nullptr;
    uint64_t bytes = 0;
    hipEvent_t done = nullptr;
    int device = -1;
    bool busy = false;        // taken by a call that has not released it yet
    bool in_flight = false;   // released with its event recorded, not yet seen complete
};

// Mapped, so the kernels of lp_compute_ragged can read a slot through its
// device pointer, and coherent (fine-grained), so no GPU cache keeps a line
// of a slot that the host refills for a later call.
constexpr unsigned kStagingFlags = hipHostMallocMapped | hipHostMallocCoherent;

static std::mutex g_staging_mutex;
static std::vector<std::unique_ptr<StagingSlot>> g_staging;
// Slots in flight, one queue per (device, stream) in the order their events
// were recorded.  Work on one stream completes in that order, so a call
// retires the finished slots from the front of each queue with one event
// query each, and a queue whose front is busy holds nothing finished; a
// host that runs ahead of the GPU keeps hundreds of slots in flight, and an
// event query costs it about 0.06 us.  Should a stream handle be reused by a
// new stream, its queue may hold a finished slot behind a busy one: that
// slot is retired later, never early, since every slot is retired on its
// own event.
struct InFlight {
    int device;
    hipStream_t stream;
    std::deque<StagingSlot *> slots;
};
static std::vector<InFlight> g_inflight;

static void retire_fronts() {
    for (auto q = g_inflight.begin(); q != g_inflight.end();) {
        while (!q->slots.empty() && hipEventQuery(q->slots.front()->done) == hipSuccess) {
            q->slots.front()->in_flight = false;
            q->slots.pop_front();
        }
        if (q->slots.empty())
            q = g_inflight.erase(q);   // streams come and go: keep only busy queues
        else
            ++q;
    }
}

// A free slot of at least `bytes` on `device` (the smallest such), a finished
// smaller one grown to `bytes`, or a new one.
static lp_status staging_acquire(uint64_t bytes, int device, StagingSlot **out) {
    std::lock_guard<std::mutex> lock(g_staging_mutex);
    retire_fronts();
    StagingSlot *fit = nullptr, *small = nullptr;
    auto pick = [&]() {
        fit = small = nullptr;
        for (auto &up : g_staging) {
            StagingSlot *sl = up.get();
            if (sl->busy || sl->in_flight || sl->device != device) continue;
            if (sl->bytes >= bytes) {
                if (fit == nullptr || sl->bytes < fit->bytes) fit = sl;
            } else if (small == nullptr) {
                small = sl;
            }
        }
    };
    pick();
    if (fit == nullptr && small != nullptr) {
        void *h = nullptr;
        LP_HIP_TRY(hipHostMalloc(&h, bytes, kStagingFlags));
        (void)hipHostFree(small->host);
        small->host = h;
        small->bytes = bytes;
        fit = small;
    }
    if (fit == nullptr) {
        std::unique_ptr<StagingSlot> sl(new (std::nothrow) StagingSlot());
        if (!sl) return LP_ERR_NOMEM;
        try {
            g_staging.reserve(g_staging.size() + 1);   // the push below cannot throw then
        } catch (...) {
            return LP_ERR_NOMEM;
        }
        LP_HIP_TRY(hipHostMalloc(&sl->host, bytes, kStagingFlags));
        const hipError_t e = hipEventCreateWithFlags(&sl->done, hipEventDisableTiming);
        if (e != hipSuccess) {
            (void)hipHostFree(sl->host);
            g_last_hip_error = int(e);
            return LP_ERR_HIP;
        }
        sl->bytes = bytes;
        sl->device = device;
        fit = sl.get();
        g_staging.push_back(std::move(sl));
    }
    fit->busy = true;
    *out = fit;
    return LP_OK;
}

// Gives a slot back.  `recorded`: its event was recorded on `stream` after
// the last work that reads it, so it joins that stream's in-flight queue;
// otherwise nothing was enqueued on it since it was taken and it is free at
// once.
static void staging_release(StagingSlot *sl, bool recorded, hipStream_t stream) {
    std::lock_guard<std::mutex> lock(g_staging_mutex);
    if (recorded) {
        try {
            InFlight *q = nullptr;
            for (auto &f : g_inflight)
                if (f.device == sl->device && f.stream == stream) q = &f;
            if (q == nullptr) {
                g_inflight.push_back(InFlight{sl->device, stream, {}});
                q = &g_inflight.back();
            }
            q->slots.push_back(sl);
        } catch (...) {
            return;   // no room to track it: it stays taken for good
        }
        sl->in_flight = true;
    }
    sl->busy = false;
}

// lp_compute_ragged lets the kernels read the descriptors of plans up to
// this many output rows (4 MiB) straight from the pinned staging slot; past
// it, a slot of that size for every call in flight would hold too much
// pinned memory, and the descriptors are uploaded instead.  In place was
// faster at every size measured, the workgroups of rows found through their
// descriptors waiting on a PCIe read included (per call, same box: 34637
// direct rows of 151936 3038.7 -> 3018.3 us, 36175 mixed-echo rows of 32000
// 634.1 -> 607.8 us).
constexpr uint64_t kZeroCopyMaxRows = 262144;

lp_status launch_checks(const lp_plan *plan, const float *logits, const float *next_token_logits,
                        const float *out_logprobs, const uint32_t *out_token_ids,
                        const void *workspace, uint64_t workspace_bytes);
lp_status launch_rows(const lp_plan &p, const float *logits, const float *next_token_logits,
                      float *out_logprobs, uint32_t *out_token_ids, void *workspace,
                      const void *desc, hipStream_t s, hipEvent_t stop = nullptr);

// One kernel launch; `stop`, when given, is recorded as the kernel ends
// through the launch's own completion signal.  A separate hipEventRecord
// after the kernel puts a marker between it and the next launch on the
// stream, which cost about 3 us per call on back-to-back launches of a
// 128 MB read (22.3 -> 25.3 us); the launch's stop event cost nothing there.
template <typename Kernel, typename... Args>
static void launch_one(Kernel kernel, dim3 grid, dim3 block, hipStream_t s, hipEvent_t stop,
                       Args... args) {
    if (stop != nullptr)
        hipExtLaunchKernelGGL(kernel, grid, block, 0, s, nullptr, stop, 0, args...);
    else
        hipLaunchKernelGGL(kernel, grid, block, 0, s, args...);
}

template <int kK, int kWaves, int kDepth>
static void launch_shape(bool direct, bool dyn, dim3 grid, hipStream_t s, hipEvent_t stop,
                         const dev::RowArgs &ra) {
    const dim3 block(kWaves * 64);
    if (direct) {
        if (dyn) launch_one(dev::row_kernel<kK, kWaves, kDepth, true, true>, grid, block, s, stop, ra);
        else launch_one(dev::row_kernel<kK, kWaves, kDepth, true, false>, grid, block, s, stop, ra);
    } else {
        if (dyn) launch_one(dev::row_kernel<kK, kWaves, kDepth, false, true>, grid, block, s, stop, ra);
        else launch_one(dev::row_kernel<kK, kWaves, kDepth, false, false>, grid, block, s, stop, ra);
    }
}

// What one call enqueues: the row kernel (rows or records), the merge
// kernel, or both.
enum class Launch { kRows, kRecords, kMerge, kRecordsThenMerge };

// `stop`, when given, goes with the last kernel enqueued.
template <int kK>
static void launch_k(const lp_plan &p, Launch what, dim3 grid, hipStream_t s, hipEvent_t stop,
                     const dev::RowArgs &ra, const dev::MergeArgs &ma, uint32_t waves,
                     uint32_t depth) {
    const bool merge = what == Launch::kMerge || what == Launch::kRecordsThenMerge;
    if (what != Launch::kMerge) {
        const bool deep = depth == 2, direct = p.direct_rows != 0, dyn = p.dynamic_chunks != 0;
        const hipEvent_t rs = merge ? nullptr : stop;
        if (waves == 16) {
            if (deep) launch_shape<kK, 16, 2>(direct, dyn, grid, s, rs, ra);
            else launch_shape<kK, 16, 1>(direct, dyn, grid, s, rs, ra);
        } else if (waves == 8) {
            if (deep) launch_shape<kK, 8, 2>(direct, dyn, grid, s, rs, ra);
            else launch_shape<kK, 8, 1>(direct, dyn, grid, s, rs, ra);
        } else {
            if (deep) launch_shape<kK, 4, 2>(direct, dyn, grid, s, rs, ra);
            else launch_shape<kK, 4, 1>(direct, dyn, grid, s, rs, ra);
        }
    }
    if (merge) {
        const uint32_t mblocks = static_cast<uint32_t>((p.out_rows + 3) / 4);
        launch_one(dev::merge_kernel<kK>, dim3(mblocks), dim3(256), s, stop, ma);
    }
}

// The kernels for the plan's slot count; false if the library is not built
// for it.
static bool launch_for_slots(const lp_plan &p, Launch what, dim3 grid, hipStream_t s,
                             const dev::RowArgs &ra, const dev::MergeArgs &ma, uint32_t waves,
                             uint32_t depth, hipEvent_t stop = nullptr) {
    switch (p.slots) {
        case 1: launch_k<1>(p, what, grid, s, stop, ra, ma, waves, depth); return true;
        case 3: launch_k<3>(p, what, grid, s, stop, ra, ma, waves, depth); return true;
        case 7: launch_k<7>(p, what, grid, s, stop, ra, ma, waves, depth); return true;
        case 15: launch_k<15>(p, what, grid, s, stop, ra, ma, waves, depth); return true;
        case 31: launch_k<31>(p, what, grid, s, stop, ra, ma, waves, depth); return true;
        case 63: launch_k<63>(p, what, grid, s, stop, ra, ma, waves, depth); return true;
        default: return false;
    }
}

// Plans that read no row: every entry of the (R, C) outputs is padding.
static lp_status launch_padding(const lp_plan &p, float *out_lp, uint32_t *out_id, hipStream_t s,
                                hipEvent_t stop = nullptr) {
    const uint64_t n = p.out_rows * p.columns;
    uint64_t g = (n + 255) / 256;
    if (g > 4096) g = 4096;
    launch_one(dev::pad_kernel, dim3(static_cast<uint32_t>(g)), dim3(256), s, stop, out_lp, out_id,
               n);
    LP_HIP_TRY(hipGetLastError());
    return LP_OK;
}

static dev::RowArgs row_args(const lp_plan &p, const float *src, uint32_t row_len, uint32_t id_base,
                             uint32_t split, const void *workspace) {
    dev::RowArgs ra{};
    ra.src = src;
    ra.row_len = row_len;
    ra.id_base = id_base;
    ra.split = split;
    ra.seg_len = static_cast<uint32_t>(segment_length(row_len, split));
    ra.out_rows = static_cast<uint32_t>(p.out_rows);
    ra.desc = static_cast<const RowDesc *>(workspace);
    return ra;
}

static lp_status check_workspace(const lp_plan *plan, const void *ws, uint64_t ws_bytes) {
    if (ws == nullptr || ws_bytes < plan->workspace_bytes) return LP_ERR_WORKSPACE;
    if ((reinterpret_cast<uintptr_t>(ws) & 255u) != 0) return LP_ERR_WORKSPACE;
    return LP_OK;
}

// ------------------------------------------------------------------ no-allocation path
//
// For callers that cannot allocate: the workspace (descriptors, then split
// records) lives in a fixed device array of kNoAllocScratchBytes, `scratch`
// below, one copy per GPU the library runs on; the descriptors are built in a
// fixed host array of the same size and sent from there, in the arguments of
// upload launches for plans of up to kMaxUploadLaunches of them, else by a
// synchronous copy.  In host code the
// array's name is only a stand-in: its device address comes from
// hipGetSymbolAddress, asked once per device with that device current, and is
// what the kernels and the copy receive.
constexpr uint64_t kNoAllocScratchBytes = 4ull << 20;
constexpr int kMaxDevices = 64;
// Plans of up to this many launches of dev::desc_upload_kernel (1984 rows)
// send their descriptors in kernel arguments; larger ones copy them from
// the host array synchronously.
constexpr uint64_t kMaxUploadLaunches = 8;

static std::mutex g_noalloc_mutex;                 // guards both arrays below
static void *g_scratch_dev[kMaxDevices] = {};      // device address of `scratch`, per device
alignas(256) static RowDesc g_noalloc_desc[kNoAllocScratchBytes / sizeof(RowDesc)];

}  // namespace lp

// The no-allocation path's device workspace (see above).  Nothing in it must
// start at zero: every descriptor is copied in before the kernels read it, and
// every split record is written by its row kernel before the merge reads it.
static __device__ __align__(256) unsigned char scratch[lp::kNoAllocScratchBytes];

namespace lp {

// The device address of `scratch` on `device` (the current device), asked
// once per device.  Called with g_noalloc_mutex held.
static lp_status scratch_address(int device, void **out) {
    if (device < 0 || device >= kMaxDevices) return LP_ERR_UNSUPPORTED;
    if (g_scratch_dev[device] == nullptr) {
        void *p = nullptr;
        LP_HIP_TRY(hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)));
        if (p == nullptr || (reinterpret_cast<uintptr_t>(p) & 255u) != 0) return LP_ERR_HIP;
        g_scratch_dev[device] = p;
    }
    *out = g_scratch_dev[device];
    return LP_OK;
}

}  // namespace lp

extern "C" {

int lp_last_hip_error(void) { return lp::g_last_hip_error; }

lp_status lp_stage_ragged(const lp_plan *plan, const uint32_t *tokens, const uint32_t *sampled_tokens,
                          void *workspace, uint64_t workspace_bytes, void *stream) {
    if (plan == nullptr) return LP_ERR_NULL_ARG;
    if (plan->out_rows == 0) return LP_OK;
    lp_status st = lp::check_workspace(plan, workspace, workspace_bytes);
    if (st != LP_OK) return st;
    const uint64_t bytes = plan->out_rows * sizeof(lp::RowDesc);
    hipStream_t s = static_cast<hipStream_t>(stream);
    int device = 0;
    LP_HIP_TRY(hipGetDevice(&device));
    lp::StagingSlot *slot = nullptr;
    st = lp::staging_acquire(bytes, device, &slot);
    if (st != LP_OK) return st;
    st = lp::build_descriptors(*plan, tokens, sampled_tokens, static_cast<lp::RowDesc *>(slot->host));
    hipError_t e = hipSuccess;
    if (st == LP_OK) e = hipMemcpyAsync(workspace, slot->host, bytes, hipMemcpyHostToDevice, s);
    if (st == LP_OK && e == hipSuccess) {
        e = hipEventRecord(slot->done, s);
        // A copy whose end no event marks may still be reading the slot:
        // the slot stays taken for good rather than be refilled under it.
        if (e != hipSuccess) {
            lp::g_last_hip_error = int(e);
            return LP_ERR_HIP;
        }
    }
    // recorded exactly when the copy was enqueued (a failed enqueue leaves
    // nothing reading the slot)
    lp::staging_release(slot, st == LP_OK && e == hipSuccess, s);
    if (st != LP_OK) return st;
    LP_HIP_TRY(e);
    return LP_OK;
}

lp_status lp_launch_ragged(const lp_plan *plan, const float *logits,
                           const float *next_token_logits, float *out_logprobs,
                           uint32_t *out_token_ids, void *workspace, uint64_t workspace_bytes,
                           void *stream) {
    const lp_status st = lp::launch_checks(plan, logits, next_token_logits, out_logprobs,
                                           out_token_ids, workspace, workspace_bytes);
    if (st != LP_OK || plan->out_rows == 0) return st;
    return lp::launch_rows(*plan, logits, next_token_logits, out_logprobs, out_token_ids,
                           workspace, workspace, static_cast<hipStream_t>(stream));
}

}  // extern "C"

namespace lp {

// The argument checks of lp_launch_ragged (LP_OK for a plan with no rows).
lp_status launch_checks(const lp_plan *plan, const float *logits, const float *next_token_logits,
                        const float *out_logprobs, const uint32_t *out_token_ids,
                        const void *workspace, uint64_t workspace_bytes) {
    if (plan == nullptr) return LP_ERR_NULL_ARG;
    if (plan->out_rows == 0) return LP_OK;
    if (out_logprobs == nullptr || out_token_ids == nullptr) return LP_ERR_NULL_ARG;
    if ((plan->has_logits ? logits : next_token_logits) == nullptr) return LP_ERR_NULL_ARG;
    const lp_status st = check_workspace(plan, workspace, workspace_bytes);
    if (st != LP_OK) return st;
    if (plan->out_rows * plan->split * plan->waves * 64ull >= (1ull << 32)) return LP_ERR_UNSUPPORTED;
    return LP_OK;
}

// Enqueues the row kernel (and the merge kernel for split rows) of a
// checked plan whose descriptors are at `desc` (device-readable: the
// workspace, or pinned host memory) and whose records go to the workspace.
lp_status launch_rows(const lp_plan &p, const float *logits, const float *next_token_logits,
                      float *out_logprobs, uint32_t *out_token_ids, void *workspace,
                      const void *desc, hipStream_t s, hipEvent_t stop) {
    const lp_plan *plan = &p;
    const float *src = plan->has_logits ? logits : next_token_logits;
    const uint64_t blocks = plan->out_rows * plan->split;
    if (plan->read_rows == 0) return lp::launch_padding(*plan, out_logprobs, out_token_ids, s, stop);
    const uint64_t words = plan->slots + 2;   // one record
    lp::dev::RowArgs ra = lp::row_args(*plan, src, plan->vocab, 0, plan->split, desc);
    ra.out_lp = out_logprobs;
    ra.out_id = out_token_ids;
    ra.records = plan->split > 1 ? 1u : 0u;
    ra.rec_row_stride = plan->split * words;
    ra.rec_seg_stride = words;
    ra.rec = reinterpret_cast<uint64_t *>(static_cast<char *>(workspace) + plan->desc_bytes);
    lp::dev::MergeArgs ma{};
    ma.nseg = plan->split;
    ma.out_rows = static_cast<uint32_t>(plan->out_rows);
    ma.rec_row_stride = ra.rec_row_stride;
    ma.rec_seg_stride = ra.rec_seg_stride;
    ma.desc = ra.desc;
    ma.rec = ra.rec;
    ma.out_lp = out_logprobs;
    ma.out_id = out_token_ids;
    const dim3 grid(static_cast<uint32_t>(blocks));
    const lp::Launch what = plan->split > 1 ? lp::Launch::kRecordsThenMerge : lp::Launch::kRows;
    if (!lp::launch_for_slots(*plan, what, grid, s, ra, ma, plan->waves, plan->depth, stop))
        return LP_ERR_UNSUPPORTED;
    LP_HIP_TRY(hipGetLastError());
    return LP_OK;
}

}  // namespace lp

namespace lp {

template <int kThreads>
static void launch_stream_read_shape(uint32_t loads, dim3 grid, hipStream_t s, const float *x,
                                     uint32_t row_len, uint32_t segs, float *partial) {
    const dim3 block(kThreads);
    switch (loads) {
        case 1: hipLaunchKernelGGL((lp::dev::stream_read_shape_kernel<kThreads, 1>), grid, block, 0, s, x, row_len, segs, partial); break;
        case 2: hipLaunchKernelGGL((lp::dev::stream_read_shape_kernel<kThreads, 2>), grid, block, 0, s, x, row_len, segs, partial); break;
        case 4: hipLaunchKernelGGL((lp::dev::stream_read_shape_kernel<kThreads, 4>), grid, block, 0, s, x, row_len, segs, partial); break;
        default: hipLaunchKernelGGL((lp::dev::stream_read_shape_kernel<kThreads, 8>), grid, block, 0, s, x, row_len, segs, partial); break;
    }
}

}  // namespace lp

extern "C" {

lp_status lp_compute_ragged(const lp_plan *plan, const float *logits, const float *next_token_logits,
                            const uint32_t *tokens, const uint32_t *sampled_tokens,
                            float *out_logprobs, uint32_t *out_token_ids, void *workspace,
                            uint64_t workspace_bytes, void *stream) {
    lp_status st = lp::launch_checks(plan, logits, next_token_logits, out_logprobs, out_token_ids,
                                     workspace, workspace_bytes);
    if (st != LP_OK || plan->out_rows == 0) return st;
    if (plan->out_rows > lp::kZeroCopyMaxRows) {
        st = lp_stage_ragged(plan, tokens, sampled_tokens, workspace, workspace_bytes, stream);
        if (st != LP_OK) return st;
        return lp::launch_rows(*plan, logits, next_token_logits, out_logprobs, out_token_ids,
                               workspace, workspace, static_cast<hipStream_t>(stream));
    }
    // Small plans: the kernels read the descriptors from the pinned staging
    // slot itself, and no copy precedes them (a 4 KB upload cost 5-8 us of
    // the call on decode).  The slot is free again once the kernels that
    // read it have run: its event is recorded after them.
    hipStream_t s = static_cast<hipStream_t>(stream);
    int device = 0;
    LP_HIP_TRY(hipGetDevice(&device));
    lp::StagingSlot *slot = nullptr;
    st = lp::staging_acquire(plan->out_rows * sizeof(lp::RowDesc), device, &slot);
    if (st != LP_OK) return st;
    st = lp::build_descriptors(*plan, tokens, sampled_tokens, static_cast<lp::RowDesc *>(slot->host));
    void *desc = nullptr;
    hipError_t e = hipSuccess;
    if (st == LP_OK) e = hipHostGetDevicePointer(&desc, slot->host, 0);
    if (st != LP_OK || e != hipSuccess) {   // nothing enqueued reads the slot
        lp::staging_release(slot, false, s);
        if (st != LP_OK) return st;
        LP_HIP_TRY(e);
    }
    // The slot's event goes with the last kernel's launch.  A failed launch
    // may still have enqueued a kernel that reads the slot, so the event is
    // then recorded on its own; if that fails too, kernels whose end no
    // event marks may still read the slot, and it stays taken for good
    // rather than be refilled under them.
    st = lp::launch_rows(*plan, logits, next_token_logits, out_logprobs, out_token_ids, workspace,
                         desc, s, slot->done);
    if (st == LP_OK) {
        lp::staging_release(slot, true, s);
        return LP_OK;
    }
    e = hipEventRecord(slot->done, s);
    if (e != hipSuccess) {
        lp::g_last_hip_error = int(e);
        return st != LP_OK ? st : LP_ERR_HIP;
    }
    lp::staging_release(slot, true, s);
    return st;
}

lp_status lp_compute_ragged_noalloc(const lp_plan *plan, const float *logits,
                                    const float *next_token_logits, const uint32_t *tokens,
                                    const uint32_t *sampled_tokens, float *out_logprobs,
                                    uint32_t *out_token_ids, void *stream) {
    if (plan == nullptr) return LP_ERR_NULL_ARG;
    if (plan->workspace_bytes > lp::kNoAllocScratchBytes) return LP_ERR_WORKSPACE;
    if (plan->out_rows == 0) return LP_OK;
    if (out_logprobs == nullptr || out_token_ids == nullptr) return LP_ERR_NULL_ARG;
    if ((plan->has_logits ? logits : next_token_logits) == nullptr) return LP_ERR_NULL_ARG;
    hipStream_t s = static_cast<hipStream_t>(stream);
    int device = 0;
    LP_HIP_TRY(hipGetDevice(&device));
    void *ws = nullptr;
    {
        std::lock_guard<std::mutex> lock(lp::g_noalloc_mutex);
        lp_status st = lp::scratch_address(device, &ws);
        if (st != LP_OK) return st;
        st = lp::build_descriptors(*plan, tokens, sampled_tokens, lp::g_noalloc_desc);
        if (st != LP_OK) return st;
        if (plan->out_rows <= uint64_t(lp::dev::kUploadRows) * lp::kMaxUploadLaunches) {
            // up to 248 descriptors per launch, carried in its arguments:
            // nothing waits, and the host array may be refilled at once
            lp::dev::DescUpload u;
            std::memset(&u, 0, sizeof(u));
            for (uint64_t first = 0; first < plan->out_rows; first += lp::dev::kUploadRows) {
                const uint64_t n = std::min<uint64_t>(lp::dev::kUploadRows, plan->out_rows - first);
                std::memcpy(u.d, lp::g_noalloc_desc + first, n * sizeof(lp::RowDesc));
                u.dst = static_cast<lp::RowDesc *>(ws) + first;
                u.count = static_cast<uint32_t>(n);
                hipLaunchKernelGGL(lp::dev::desc_upload_kernel, dim3(1), dim3(256), 0, s, u);
                LP_HIP_TRY(hipGetLastError());
            }
        } else {
            // the host array is not pinned: the copy is synchronous, and the
            // stream is drained before the array may be refilled
            LP_HIP_TRY(hipMemcpyWithStream(ws, lp::g_noalloc_desc,
                                           plan->out_rows * sizeof(lp::RowDesc),
                                           hipMemcpyHostToDevice, s));
            LP_HIP_TRY(hipStreamSynchronize(s));
        }
    }
    return lp_launch_ragged(plan, logits, next_token_logits, out_logprobs, out_token_ids, ws,
                            lp::kNoAllocScratchBytes, stream);
}

lp_status lp_shard_records(const lp_plan *plan, uint32_t vocab_begin, uint32_t shard_vocab,
                           const float *shard_logits, const float *shard_next_token_logits,
                           uint64_t *records, void *workspace, uint64_t workspace_bytes,
                           void *stream) {
    if (plan == nullptr) return LP_ERR_NULL_ARG;
    if (shard_vocab < 1 || uint64_t(vocab_begin) + shard_vocab > plan->vocab) return LP_ERR_SHAPE;
    if (shard_vocab > lp::kMaxSegment) return LP_ERR_UNSUPPORTED;
    if (plan->out_rows == 0 || plan->read_rows == 0) return LP_OK;
    const float *src = plan->has_logits ? shard_logits : shard_next_token_logits;
    if (src == nullptr || records == nullptr) return LP_ERR_NULL_ARG;
    lp_status st = lp::check_workspace(plan, workspace, workspace_bytes);
    if (st != LP_OK) return st;
    uint32_t waves = 0, depth = 0;
    lp::shard_shape(*plan, shard_vocab, &waves, &depth);
    if (plan->out_rows * waves * 64ull >= (1ull << 32)) return LP_ERR_UNSUPPORTED;
    hipStream_t s = static_cast<hipStream_t>(stream);
    lp::dev::RowArgs ra = lp::row_args(*plan, src, shard_vocab, vocab_begin, 1, workspace);
    ra.records = 1;
    ra.rec_row_stride = plan->slots + 2;
    ra.rec_seg_stride = 0;
    ra.rec = records;
    lp::dev::MergeArgs ma{};
    const dim3 grid(static_cast<uint32_t>(plan->out_rows));
    if (!lp::launch_for_slots(*plan, lp::Launch::kRecords, grid, s, ra, ma, waves, depth))
        return LP_ERR_UNSUPPORTED;
    LP_HIP_TRY(hipGetLastError());
    return LP_OK;
}

lp_status lp_merge_shards(const lp_plan *plan, uint32_t num_shards, const uint64_t *records,
                          float *out_logprobs, uint32_t *out_token_ids, void *workspace,
                          uint64_t workspace_bytes, void *stream) {
    if (plan == nullptr) return LP_ERR_NULL_ARG;
    if (num_shards < 1 || num_shards > lp::kMaxSplit ||
        uint64_t(num_shards) * plan->slots > lp::kMaxMergeKeys)
        return LP_ERR_UNSUPPORTED;
    if (plan->out_rows == 0) return LP_OK;
    if (out_logprobs == nullptr || out_token_ids == nullptr) return LP_ERR_NULL_ARG;
    lp_status st = lp::check_workspace(plan, workspace, workspace_bytes);
    if (st != LP_OK) return st;
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (plan->read_rows == 0) return lp::launch_padding(*plan, out_logprobs, out_token_ids, s);
    if (records == nullptr) return LP_ERR_NULL_ARG;
    const uint64_t words = plan->slots + 2;
    lp::dev::RowArgs ra{};
    lp::dev::MergeArgs ma{};
    ma.nseg = num_shards;
    ma.out_rows = static_cast<uint32_t>(plan->out_rows);
    ma.rec_row_stride = words;
    ma.rec_seg_stride = plan->out_rows * words;
    ma.desc = static_cast<const lp::RowDesc *>(workspace);
    ma.rec = records;
    ma.out_lp = out_logprobs;
    ma.out_id = out_token_ids;
    if (!lp::launch_for_slots(*plan, lp::Launch::kMerge, dim3(1), s, ra, ma, plan->waves, plan->depth))
        return LP_ERR_UNSUPPORTED;
    LP_HIP_TRY(hipGetLastError());
    return LP_OK;
}

lp_status lp_bench_stream_read_shape(const float *x, uint32_t rows, uint32_t row_len,
                                     uint32_t segments, uint32_t threads, uint32_t loads,
                                     float *partial_out, void *stream) {
    if (rows == 0) return LP_OK;
    if (x == nullptr || partial_out == nullptr) return LP_ERR_NULL_ARG;
    if ((reinterpret_cast<uintptr_t>(x) & 15u) != 0 || (row_len & 3u) != 0 || row_len == 0)
        return LP_ERR_UNSUPPORTED;
    if (segments < 1 || segments > 64 || uint64_t(rows) * segments >= (1ull << 31))
        return LP_ERR_UNSUPPORTED;
    if (loads != 1 && loads != 2 && loads != 4 && loads != 8) return LP_ERR_UNSUPPORTED;
    const dim3 grid(rows * segments);
    hipStream_t s = static_cast<hipStream_t>(stream);
    switch (threads) {
        case 256: lp::launch_stream_read_shape<256>(loads, grid, s, x, row_len, segments, partial_out); break;
        case 512: lp::launch_stream_read_shape<512>(loads, grid, s, x, row_len, segments, partial_out); break;
        case 1024: lp::launch_stream_read_shape<1024>(loads, grid, s, x, row_len, segments, partial_out); break;
        default: return LP_ERR_UNSUPPORTED;
    }
    LP_HIP_TRY(hipGetLastError());
    return LP_OK;
}

lp_status lp_bench_stream_read(const float *x, uint32_t rows, uint32_t row_len, float *partial_out,
                               void *stream) {
    if (rows == 0) return LP_OK;
    if (x == nullptr || partial_out == nullptr) return LP_ERR_NULL_ARG;
    if ((reinterpret_cast<uintptr_t>(x) & 15u) != 0 || (row_len & 3u) != 0 || row_len == 0)
        return LP_ERR_UNSUPPORTED;
    hipLaunchKernelGGL(lp::dev::stream_read_kernel, dim3(rows), dim3(512), 0,
                       static_cast<hipStream_t>(stream), x, row_len, partial_out);
    LP_HIP_TRY(hipGetLastError());
    return LP_OK;
}

}  // extern "C"
