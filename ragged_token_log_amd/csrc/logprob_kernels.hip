// Device code and launch glue for ragged batched token log-probabilities on
// CDNA4 (gfx950, wave64).
//
// What is computed follows [MAX] "MAX Python SDK 中 log_probabilities 模块解析：
// ragged 批量 Token 对数概率的计算图构建与执行" (§log_probabilities_ragged_graph:
// per output row, 7 ranked slots plus one slot for the chosen token; §图支持的
// 最大 top-n: top_n <= 7) and [SGL] "logprob、finish reason 与 output
// processing" (§logprob 的数值形态: a logprob is log p, so <= 0).  The pages keep
// the 7 candidates in a min-heap; this file does not.  On gfx950 the work is an
// HBM stream with a few VALU ops per element, so the design aims at reading
// each logit exactly once with 16-byte loads and doing as little per element
// as possible:
//
//  * Each row (or row segment) is one workgroup of 4, 8 or 16 waves.  Waves
//    take interleaved chunks of 64 lanes x kU float4, read with nontemporal
//    buffer loads, two chunks in flight per wave.  Per chunk a lane reduces
//    its 16 values to a chunk max and updates a running (m, s) with
//    s = sum e^(x-m) (exp2 with log2(e) applied after an exact subtraction).
//  * Ranking uses a 64-bit order key: the fp32 bits mapped to an unsigned
//    order (with -0.0 folded onto +0.0) in the high word, the complemented
//    token id in the low word.  A larger key is a better (value, id) pair, so
//    ties go to the lowest id and every merge uses one total order.
//  * The workgroup keeps one shared list of the 7 best keys entered so far in
//    LDS, filled by cascades of atomic max operations, and every wave filters
//    its chunks against one bound T: a seed taken from all waves' first
//    chunks (one barrier), raised to the list's 7th key as it fills.  A chunk
//    whose lane maxima stay below T costs one compare; the few columns that
//    beat it enter their keys one at a time.
//  * The waves' (m, s) pairs merge through LDS; the last wave to finish
//    writes lp = x - (m + ln s) for the 7 listed keys and the chosen token.
//  * With too few rows to fill 256 CUs, a row is split into segments, one
//    workgroup each, which write (m, s, 7 keys) records; a second kernel (one
//    wave per row) merges a row's records in segment order and writes it.
//
// No MFMA: there is no contraction here.
#include <hip/hip_runtime.h>

#include <cstdint>
#include <cstring>

#include "lp_internal.h"

namespace lp {
namespace dev {

constexpr int kWave = 64;
constexpr int kU = 4;                // float4 loads per lane per chunk
constexpr int kChunkF4 = kWave * kU; // float4 per wave-chunk (1024 elements)
constexpr int kSlots = int(kTopSlots);
constexpr float kLog2e = 1.4426950408889634f;

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

__device__ __forceinline__ float wave_max_f32(float v) {
    v = fmaxf(v, dpp_f32<kDppXor1>(v));
    v = fmaxf(v, dpp_f32<kDppXor2>(v));
    v = fmaxf(v, dpp_f32<kDppHalfMirror>(v));
    v = fmaxf(v, dpp_f32<kDppMirror>(v));
    return fmaxf(fmaxf(readlane_f32(v, 0), readlane_f32(v, 16)),
                 fmaxf(readlane_f32(v, 32), readlane_f32(v, 48)));
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

// Lane 0 adds 1 to an LDS counter; every lane gets the previous value.
__device__ __forceinline__ uint32_t lds_arrive(uint32_t *counter, int lane) {
    uint32_t prev = 0;
    if (lane == 0) prev = __hip_atomic_fetch_add(counter, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
    return readlane_u32(prev, 0);
}

// Logits are read exactly once: nontemporal 16-byte loads (the `nt` form of
// buffer_load_dwordx4) stream them without displacing reusable cache lines;
// on gfx950 they sustain ~13% more HBM bandwidth than plain loads here.
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

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
__device__ __forceinline__ void lse_merge(float &m, float &s, float m2, float s2) {
    const float M = fmaxf(m, m2);
    const float Ms = (M == -INFINITY) ? 0.0f : M;
    s = s * fast_exp2((m - Ms) * kLog2e) + s2 * fast_exp2((m2 - Ms) * kLog2e);
    m = M;
}

template <int kCtrl>
__device__ __forceinline__ void lse_dpp_step(float &m, float &s) {
    const float m2 = dpp_f32<kCtrl>(m);
    const float s2 = dpp_f32<kCtrl>(s);
    lse_merge(m, s, m2, s2);
}

// Every lane ends with the wave's (m, s), merged in a fixed order.
__device__ __forceinline__ void wave_lse(float &m, float &s) {
    lse_dpp_step<kDppXor1>(m, s);
    lse_dpp_step<kDppXor2>(m, s);
    lse_dpp_step<kDppHalfMirror>(m, s);
    lse_dpp_step<kDppMirror>(m, s);
    float M = readlane_f32(m, 0), S = readlane_f32(s, 0);
    lse_merge(M, S, readlane_f32(m, 16), readlane_f32(s, 16));
    float M2 = readlane_f32(m, 32), S2 = readlane_f32(s, 32);
    lse_merge(M2, S2, readlane_f32(m, 48), readlane_f32(s, 48));
    lse_merge(M, S, M2, S2);
    m = M;
    s = S;
}

// Best 7 keys of up to kPer*64 keys held kPer per lane (0 = empty).  Returns,
// in lane r < 7, the r-th best key (0 if fewer exist); *count gets how many
// were found.  Each round finds the largest high word across the wave, then
// the largest low word among keys with that high word (keys are unique).
template <int kPer>
__device__ __forceinline__ uint64_t wave_select7(uint64_t (&e)[kPer], int lane, uint32_t *count) {
    uint64_t mine = 0;
    uint32_t found = 0;
#pragma unroll 1
    for (int r = 0; r < kSlots; ++r) {
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

// ------------------------------------------------------------------ candidates
//
// A workgroup keeps one list of the 7 best keys entered so far, in LDS slots
// (descending; 0 = empty).  A key enters by a cascade of atomic max
// operations down the slots: at each slot the atomic leaves the larger of
// (slot, key) there and hands the smaller on to the next slot.  Every key
// visits the slots in order and a slot keeps the largest key that ever
// reached it, so whatever the interleaving of the waves' cascades, slot i ends
// with the (i+1)-th best of all keys entered, and at every moment the slots
// are in descending order.  A key handed on at or below a bound T that 7
// other real keys exceed can be dropped.  All waves filter against one bound,
// T = max(seed, slot 6): the seed comes from the first chunks' lane maxima,
// slot 6 is the 7th best key entered so far.

// The smallest value a key above T can have; a cheap superset test for
// candidates (below the key of -inf, nothing is excluded).
__device__ __forceinline__ float threshold_value(uint64_t T) {
    return uint32_t(T >> 32) >= 0x007FFFFFu ? key_value(T) : -INFINITY;
}

// Enters the lanes' keys that are above T (a lane passes 0 to enter none)
// and returns a bound at least T.  Keys go one at a time, as wave-uniform
// values, each with one atomic per slot it moves through.  Slots only ever
// grow, so a key below what a slot held at a snapshot would pass that slot
// unchanged: a key starts at the first slot the snapshot had below it,
// mostly the last one.  After a key settles in the last slot, that slot
// holds at least the larger of its old value and the key, which bounds the
// later keys.
__device__ __forceinline__ uint64_t enter_keys(uint64_t *slots, uint64_t k, uint64_t T, int lane) {
    uint64_t live = __ballot(k > T);
    if (live == 0) return T;
    const uint64_t held = lds_load_relaxed(slots + (lane < kSlots ? lane : kSlots - 1));
    const bool slot_lane = lane < kSlots;
    while (live != 0) {
        const int l = __builtin_ctzll(live);
        live &= live - 1;
        uint64_t kk = readlane_u64(k, l);
        if (kk <= T) continue;
        uint32_t i = uint32_t(__popcll(__ballot(slot_lane && held > kk)));
        for (; i < uint32_t(kSlots); ++i) {
            uint64_t old = 0;
            if (lane == 0)
                old = __hip_atomic_fetch_max(slots + i, kk, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
            old = readlane_u64(old, 0);
            if (i == uint32_t(kSlots - 1)) T = umax64(T, umax64(old, kk));
            if (old < kk) {
                kk = old;             // the slot took the key; the old one moves on
                if (kk <= T) break;
            }
        }
    }
    return T;
}

__device__ __forceinline__ float f4_get(const f32x4 &v, int q) {
    return q == 0 ? v.x : q == 1 ? v.y : q == 2 ? v.z : v.w;
}

// A bound from one real element per lane (or -inf for none): if 7 lanes hold
// values >= t (counting lanes that tie), no element below t can be in the
// top 7, so the bound may be just under the smallest key of value t.  A -inf
// t excludes nothing.
__device__ __forceinline__ uint64_t bound_from_lane_values(float v) {
    float t = -INFINITY;
    uint32_t cnt = 0;
#pragma unroll 1
    for (int r = 0; r < kSlots; ++r) {
        const float mx = wave_max_f32(v);
        cnt += uint32_t(__popcll(__ballot(v == mx)));
        t = mx;
        if (cnt >= uint32_t(kSlots)) break;
        v = (v == mx) ? -INFINITY : v;
    }
    if (cnt < uint32_t(kSlots)) return 0ull;
    const uint64_t k = order_key(t, kPadId);  // low word 0: smallest key of value t
    return k > 0 ? k - 1 : 0ull;
}

// ------------------------------------------------------------------ row kernel

struct RowArgs {
    const float *src;          // logits the op reads (rows of V floats)
    uint32_t vocab;
    uint32_t split;            // segments per row
    uint32_t seg_len;          // elements per segment (multiple of 4)
    uint32_t out_rows;
    const RowDesc *desc;
    float *out_lp;             // split == 1: (R, 8)
    uint32_t *out_id;          // split == 1: (R, 8)
    PartialRec *partials;      // split > 1: (R, split)
};

__device__ __forceinline__ void write_row(float *out_lp, uint32_t *out_id, uint64_t o, int lane,
                                          uint64_t key, uint32_t top_n, float lse,
                                          float x_chosen, uint32_t chosen) {
    // lanes 0..6: ranked slots; lane 7: the chosen token
    if (lane < kSlots) {
        const bool valid = uint32_t(lane) < top_n && key != 0;
        out_lp[o * kCols + lane] = valid ? key_value(key) - lse : -INFINITY;
        out_id[o * kCols + lane] = valid ? key_id(key) : kPadId;
    } else if (lane == kSlots) {
        out_lp[o * kCols + lane] = x_chosen - lse;
        out_id[o * kCols + lane] = chosen;
    }
}

// The whole descriptor of a workgroup's row in one 16-byte scalar load (not
// one dependent load per field as they are first used).
__device__ __forceinline__ RowDesc load_desc_uniform(const RowDesc *desc, uint32_t o) {
    uint4 v = *reinterpret_cast<const uint4 *>(desc + o);
    asm volatile("" : "+s"(v.x), "+s"(v.y), "+s"(v.z));
    return RowDesc{v.x, v.y, v.z, v.w};
}

__device__ __forceinline__ void write_padding(float *out_lp, uint32_t *out_id, uint64_t o, int lane) {
    if (lane < int(kCols)) {
        out_lp[o * kCols + lane] = -INFINITY;
        out_id[o * kCols + lane] = kPadId;
    }
}

template <int kWaves, int kDepth>
__global__ __launch_bounds__(kWaves * kWave) void row_kernel(RowArgs a) {
    constexpr int kThreads = kWaves * kWave;
    __shared__ uint64_t s_top[kSlots];
    __shared__ float s_lmax[kWaves * kWave];
    __shared__ float s_m[kWaves], s_s[kWaves];
    __shared__ uint32_t s_done;

    const int tid = int(threadIdx.x);
    const int lane = tid & (kWave - 1);
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: loop control stays scalar
    const uint32_t o = blockIdx.x / a.split;
    const uint32_t seg = blockIdx.x - o * a.split;
    const RowDesc d = load_desc_uniform(a.desc, o);

    if (d.top_n == 0) {  // padding-only row: no logits read (the merge kernel pads split rows)
        if (a.split == 1 && wave == 0) write_padding(a.out_lp, a.out_id, o, lane);
        return;
    }

    const uint32_t V = a.vocab;
    const float *row = a.src + uint64_t(d.src_row) * V;
    const uint64_t seg_start = uint64_t(seg) * a.seg_len;
    const uint32_t v0 = seg_start < V ? uint32_t(seg_start) : V;
    const uint32_t v1 = (uint64_t(v0) + a.seg_len < V) ? v0 + a.seg_len : V;

    float m = -INFINITY, s = 0.0f;  // this lane's running max and sum of e^(x - m)
    float x_chosen;
    // wave-uniform filter state: seed bound, T = max(seed, slot 6), T's value
    uint64_t seed = 0, T = 0;
    float tv = -INFINITY;
    auto refresh = [&]() __attribute__((always_inline)) {
        T = umax64(seed, uniform64(lds_load_relaxed(&s_top[kSlots - 1])));
        tv = threshold_value(T);
    };

    // aligned body: float4 loads from a 16-byte aligned element a0
    uint32_t a0 = v0;
    {
        const uint32_t mis = uint32_t((reinterpret_cast<uintptr_t>(row + v0) >> 2) & 3u);
        a0 = v0 + ((4u - mis) & 3u);
        if (a0 > v1) a0 = v1;
    }
    const uint32_t nf4 = (v1 - a0) >> 2;
    const uint32_t nchunks = nf4 / uint32_t(kChunkF4);

    // The body's full chunks are read through a buffer resource whose range
    // ends after the last of them: a load of a chunk past the end returns
    // zeros without touching memory.  So every refill is unconditional, no
    // buffer value ever merges two paths, and the compiler keeps each buffer
    // in place instead of copying buffers at the loop's back edge (a copy
    // would first wait for every load in flight).
    const StreamRange body = make_stream_range(row + a0, nchunks * uint32_t(kChunkF4 * 16));
    auto load_chunk = [&](f32x4 (&x)[kU], uint32_t ch) __attribute__((always_inline)) {
        const uint32_t off = ch * uint32_t(kChunkF4 * 16) + uint32_t(lane) * 16u;
#pragma unroll
        for (int u = 0; u < kU; ++u) x[u] = stream_load(body, off + uint32_t(u * kWave * 16));
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

    // LSE update for one chunk; returns the lane's chunk max
    auto lse_chunk = [&](const f32x4 (&x)[kU]) __attribute__((always_inline)) {
        float cm = fmaxf(fmaxf(x[0].x, x[0].y), fmaxf(x[0].z, x[0].w));
#pragma unroll
        for (int u = 1; u < kU; ++u)
            cm = fmaxf(cm, fmaxf(fmaxf(x[u].x, x[u].y), fmaxf(x[u].z, x[u].w)));
        const float mn = fmaxf(m, cm);
        const float ms = (mn == -INFINITY) ? 0.0f : mn;
        float acc[kU];
#pragma unroll
        for (int u = 0; u < kU; ++u) {
            acc[u] = fast_exp2((x[u].x - ms) * kLog2e) + fast_exp2((x[u].y - ms) * kLog2e) +
                     (fast_exp2((x[u].z - ms) * kLog2e) + fast_exp2((x[u].w - ms) * kLog2e));
        }
        float csum = acc[0];
#pragma unroll
        for (int u = 1; u < kU; ++u) csum += acc[u];
        s = s * fast_exp2((m - ms) * kLog2e) + csum;
        m = mn;
        return cm;
    };

    // Top-k part for one chunk whose lane maxima are cm, against the bound
    // as of this chunk.  A float compare of the lane maxima with T's value
    // passes almost every chunk by; then the order key of (lane max, the
    // lane's first id), which no key of the lane's chunk exceeds; then one
    // float compare per column, and the columns with candidates cascade.
    auto topk_chunk = [&](const f32x4 (&x)[kU], uint32_t ch, float cm) __attribute__((always_inline)) {
        if (__ballot(cm >= tv) == 0) return;
        const uint32_t first_id = a0 + 4u * (ch * uint32_t(kChunkF4) + uint32_t(lane));
        if (__ballot(order_key(cm, first_id) > T) == 0) return;
        // columns (u, q) holding a candidate, then one column at a time
        // through a single copy of the entry code (uniform register indexing)
        static_assert(kU == 4, "16 columns per chunk");
        uint32_t cols = 0;
#pragma unroll
        for (int u = 0; u < kU; ++u) {
            const float gm = fmaxf(fmaxf(x[u].x, x[u].y), fmaxf(x[u].z, x[u].w));
            if (__ballot(gm >= tv) == 0) continue;
#pragma unroll
            for (int q = 0; q < 4; ++q)
                cols |= (__ballot(f4_get(x[u], q) >= tv) != 0 ? 1u : 0u) << (4 * u + q);
        }
        const f32x16 xv = __builtin_shufflevector(__builtin_shufflevector(x[0], x[1], 0, 1, 2, 3, 4, 5, 6, 7),
                                                  __builtin_shufflevector(x[2], x[3], 0, 1, 2, 3, 4, 5, 6, 7),
                                                  0, 1, 2, 3, 4, 5, 6, 7, 8, 9, 10, 11, 12, 13, 14, 15);
        while (cols != 0) {
            const uint32_t j = uint32_t(__builtin_ctz(cols));
            cols &= cols - 1;
            const uint32_t id = first_id + 4u * uint32_t(kWave) * (j >> 2) + (j & 3u);
            T = enter_keys(s_top, order_key(xv[j], id), T, lane);
        }
        tv = threshold_value(T);
    };

    // The bound is re-read from LDS for every chunk, the read issued before
    // the chunk's arithmetic so that its latency hides there.
    auto process_chunk = [&](const f32x4 (&x)[kU], uint32_t ch) __attribute__((always_inline)) {
        const uint64_t s6 = lds_load_relaxed(&s_top[kSlots - 1]);
        const float cm = lse_chunk(x);
        T = umax64(seed, uniform64(s6));
        tv = threshold_value(T);
        topk_chunk(x, ch, cm);
    };

    // kDepth chunks in flight per wave (register buffers used in rotation).
    // After the first chunk every wave publishes its lanes' chunk maxima; past
    // one barrier each wave takes, per lane position, the max over the waves
    // and seeds the threshold from the 7th largest of those 64 values, so all
    // waves start from the same bound for the whole workgroup's first chunks.
    {
        f32x4 xb[kDepth][kU];
        uint32_t ch = uint32_t(wave);
#pragma unroll
        for (int d = 0; d < kDepth; ++d)
            refill(xb[d], ch + uint32_t(d * kWaves));
        // the chosen token's logit, fetched now so that its latency hides under
        // the stream instead of trailing the final merge (a per-lane index keeps
        // it a vector load that nothing waits on before its use)
        x_chosen = row[(a.split == 1 && lane == kSlots) ? d.chosen : 0u];
        if (tid < kSlots) s_top[tid] = 0;
        if (tid == 0) s_done = 0;
        float cm0 = -INFINITY;
        if (ch < nchunks) cm0 = lse_chunk(xb[0]);
        s_lmax[wave * kWave + lane] = cm0;
        __syncthreads();
        {
            float cmx = s_lmax[lane];
#pragma unroll
            for (int i = 1; i < kWaves; ++i) cmx = fmaxf(cmx, s_lmax[i * kWave + lane]);
            seed = bound_from_lane_values(cmx);
            T = seed;
            tv = threshold_value(T);
        }
        if (ch < nchunks) topk_chunk(xb[0], ch, cm0);
        constexpr uint32_t kAhead = uint32_t(kDepth * kWaves);
        refill(xb[0], ch + kAhead);
        ch += kWaves;
        // The remaining chunks of this wave go in whole rounds of kDepth steps
        // (buffer d % kDepth holds chunk ch on the d-th step of a round); in
        // the last round, steps past the end skip their chunk and their
        // refill reads nothing.  The loop has one exit, at its bottom, and no
        // buffer is read after it: an exit from the middle, or a use after
        // the loop, would add paths on which buffers are copied between
        // registers or every wait for loads in flight must be stricter.
        const uint32_t mine = nchunks > uint32_t(wave) ? (nchunks - uint32_t(wave) + kWaves - 1) / kWaves : 0u;
        const uint32_t rounds = mine > 1 ? (mine - 1 + kDepth - 1) / uint32_t(kDepth) : 0u;
        for (uint32_t r = 0; r < rounds; ++r) {
#pragma unroll
            for (int d = 1; d <= kDepth; ++d) {
                if (ch < nchunks) process_chunk(xb[d % kDepth], ch);
                refill(xb[d % kDepth], ch + kAhead);
                ch += kWaves;
            }
        }
    }

    // head (before a0) and tail (after the last full chunk): one element per
    // thread per pass
    {
        refresh();
        const uint32_t nh = a0 - v0;
        const uint32_t tail0 = a0 + nchunks * uint32_t(kChunkF4) * 4u;
        const uint32_t nrest = nh + (v1 - tail0);
        for (uint32_t base = 0; base < nrest; base += kThreads) {
            const uint32_t r = base + uint32_t(tid);
            const bool valid = r < nrest;
            const uint32_t e = (r < nh) ? v0 + r : tail0 + (r - nh);
            float x = -INFINITY;
            if (valid) x = row[e];
            const float mn = fmaxf(m, x);
            const float ms = (mn == -INFINITY) ? 0.0f : mn;
            s = s * fast_exp2((m - ms) * kLog2e) + fast_exp2((x - ms) * kLog2e);
            m = mn;
            T = enter_keys(s_top, valid ? order_key(x, e) : 0ull, T, lane);
        }
    }

    // per wave: (m, s) across lanes into LDS; the last wave of the workgroup
    // to get here merges them and writes the row (or the segment's record)
    wave_lse(m, s);
    if (lane == 0) {
        s_m[wave] = m;
        s_s[wave] = s;
    }
    lds_release();
    if (lds_arrive(&s_done, lane) != uint32_t(kWaves - 1)) return;
    lds_acquire();

    const uint64_t mine = lane < kSlots ? lds_load_relaxed(&s_top[lane < kSlots ? lane : 0]) : 0ull;
    float M = -INFINITY, S = 0.0f;
    if (lane < kWaves) {
        M = s_m[lane];
        S = s_s[lane];
    }
    wave_lse(M, S);

    if (a.split == 1) {
        write_row(a.out_lp, a.out_id, o, lane, mine, d.top_n, M + logf(S), x_chosen, d.chosen);
    } else {
        PartialRec *rec = a.partials + uint64_t(o) * a.split + seg;
        if (lane == 0) {
            rec->m = M;
            rec->s = S;
        }
        if (lane < kSlots) rec->keys[lane] = mine;
    }
}

// ------------------------------------------------------------------ merge kernel

struct MergeArgs {
    const float *src;
    uint32_t vocab;
    uint32_t split;
    uint32_t out_rows;
    const RowDesc *desc;
    const PartialRec *partials;
    float *out_lp;
    uint32_t *out_id;
};

// Split variant, second launch: one wave per output row combines the row's
// segment records in segment order, then writes the row.
__global__ __launch_bounds__(256) void merge_kernel(MergeArgs a) {
    const int lane = int(threadIdx.x) & (kWave - 1);
    const uint32_t o = blockIdx.x * 4u + (threadIdx.x >> 6);
    if (o >= a.out_rows) return;
    const RowDesc d = a.desc[o];
    if (d.top_n == 0) {
        write_padding(a.out_lp, a.out_id, o, lane);
        return;
    }
    const float *row = a.src + uint64_t(d.src_row) * a.vocab;
    const float x_chosen = lane == kSlots ? row[d.chosen] : 0.0f;
    const PartialRec *recs = a.partials + uint64_t(o) * a.split;
    float m = -INFINITY, s = 0.0f;
    if (uint32_t(lane) < a.split) {
        m = recs[lane].m;
        s = recs[lane].s;
    }
    wave_lse(m, s);
    constexpr int kPer = (int(kMaxSplit) * kSlots + kWave - 1) / kWave;
    const uint32_t nkeys = a.split * uint32_t(kSlots);
    uint64_t e[kPer];
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
        const uint32_t idx = uint32_t(lane + kWave * i);
        e[i] = idx < nkeys ? recs[idx / kSlots].keys[idx % kSlots] : 0ull;
    }
    uint32_t found;
    const uint64_t top = wave_select7<kPer>(e, lane, &found);
    write_row(a.out_lp, a.out_id, o, lane, top, d.top_n, m + logf(s), x_chosen, d.chosen);
}

// ------------------------------------------------------------------ streaming-read probe

__global__ __launch_bounds__(256) void stream_read_kernel(const float4 *x, uint64_t n4,
                                                         const float *tail, uint32_t ntail,
                                                         float *partial) {
    __shared__ float red[4];
    const uint64_t stride = uint64_t(gridDim.x) * 256u;
    float acc0 = 0.f, acc1 = 0.f;
    for (uint64_t i = uint64_t(blockIdx.x) * 256u + threadIdx.x; i < n4; i += stride) {
        const float4 v = x[i];
        acc0 += v.x + v.y;
        acc1 += v.z + v.w;
    }
    if (blockIdx.x == 0 && threadIdx.x < ntail) acc0 += tail[threadIdx.x];
    float acc = acc0 + acc1;
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) acc += __shfl_xor(acc, o);
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = acc;
    __syncthreads();
    if (threadIdx.x == 0) partial[blockIdx.x] = red[0] + red[1] + red[2] + red[3];
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

void release_staging(lp_plan &p) {
    if (p.staging_event != nullptr) {
        if (p.staging_pending) (void)hipEventSynchronize(static_cast<hipEvent_t>(p.staging_event));
        (void)hipEventDestroy(static_cast<hipEvent_t>(p.staging_event));
        p.staging_event = nullptr;
    }
    if (p.staging != nullptr) {
        (void)hipHostFree(p.staging);
        p.staging = nullptr;
    }
    p.staging_pending = false;
}

static lp_status check_workspace(const lp_plan *plan, const void *ws, uint64_t ws_bytes) {
    if (ws == nullptr || ws_bytes < plan->workspace_bytes) return LP_ERR_WORKSPACE;
    if ((reinterpret_cast<uintptr_t>(ws) & 255u) != 0) return LP_ERR_WORKSPACE;
    return LP_OK;
}

}  // namespace lp

extern "C" {

int lp_last_hip_error(void) { return lp::g_last_hip_error; }

lp_status lp_stage_ragged(lp_plan *plan, const uint32_t *tokens, const uint32_t *sampled_tokens,
                          void *workspace, uint64_t workspace_bytes, void *stream) {
    if (plan == nullptr) return LP_ERR_NULL_ARG;
    if (plan->out_rows == 0) return LP_OK;
    lp_status st = lp::check_workspace(plan, workspace, workspace_bytes);
    if (st != LP_OK) return st;
    const uint64_t bytes = plan->out_rows * sizeof(lp::RowDesc);
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (plan->staging == nullptr || plan->staging_bytes < bytes) {
        lp::release_staging(*plan);
        LP_HIP_TRY(hipHostMalloc(&plan->staging, bytes, hipHostMallocDefault));
        plan->staging_bytes = bytes;
        hipEvent_t ev;
        LP_HIP_TRY(hipEventCreateWithFlags(&ev, hipEventDisableTiming));
        plan->staging_event = ev;
    } else if (plan->staging_pending) {
        LP_HIP_TRY(hipEventSynchronize(static_cast<hipEvent_t>(plan->staging_event)));
        plan->staging_pending = false;
    }
    st = lp::build_descriptors(*plan, tokens, sampled_tokens,
                               static_cast<lp::RowDesc *>(plan->staging));
    if (st != LP_OK) return st;
    LP_HIP_TRY(hipMemcpyAsync(workspace, plan->staging, bytes, hipMemcpyHostToDevice, s));
    LP_HIP_TRY(hipEventRecord(static_cast<hipEvent_t>(plan->staging_event), s));
    plan->staging_pending = true;
    return LP_OK;
}

lp_status lp_launch_ragged(const lp_plan *plan, const float *logits,
                           const float *next_token_logits, float *out_logprobs,
                           uint32_t *out_token_ids, void *workspace, uint64_t workspace_bytes,
                           void *stream) {
    if (plan == nullptr) return LP_ERR_NULL_ARG;
    if (plan->out_rows == 0) return LP_OK;
    if (out_logprobs == nullptr || out_token_ids == nullptr) return LP_ERR_NULL_ARG;
    const float *src = plan->has_logits ? logits : next_token_logits;
    if (src == nullptr) return LP_ERR_NULL_ARG;
    lp_status st = lp::check_workspace(plan, workspace, workspace_bytes);
    if (st != LP_OK) return st;
    const uint32_t waves = plan->waves;
    const uint64_t blocks = plan->out_rows * plan->split;
    if (blocks * waves * 64ull >= (1ull << 32)) return LP_ERR_UNSUPPORTED;

    char *ws = static_cast<char *>(workspace);
    auto *desc = reinterpret_cast<const lp::RowDesc *>(ws);
    auto *partials = reinterpret_cast<lp::PartialRec *>(ws + plan->desc_bytes);
    lp::dev::RowArgs ra;
    ra.src = src;
    ra.vocab = plan->vocab;
    ra.split = plan->split;
    ra.seg_len = static_cast<uint32_t>(lp::segment_length(plan->vocab, plan->split));
    ra.out_rows = static_cast<uint32_t>(plan->out_rows);
    ra.desc = desc;
    ra.out_lp = out_logprobs;
    ra.out_id = out_token_ids;
    ra.partials = partials;
    hipStream_t s = static_cast<hipStream_t>(stream);
    const dim3 grid(static_cast<uint32_t>(blocks));
    const bool deep = plan->depth == 4;
    if (waves == 16) {
        if (deep) hipLaunchKernelGGL((lp::dev::row_kernel<16, 4>), grid, dim3(16 * 64), 0, s, ra);
        else hipLaunchKernelGGL((lp::dev::row_kernel<16, 2>), grid, dim3(16 * 64), 0, s, ra);
    } else if (waves == 8) {
        if (deep) hipLaunchKernelGGL((lp::dev::row_kernel<8, 4>), grid, dim3(8 * 64), 0, s, ra);
        else hipLaunchKernelGGL((lp::dev::row_kernel<8, 2>), grid, dim3(8 * 64), 0, s, ra);
    } else {
        if (deep) hipLaunchKernelGGL((lp::dev::row_kernel<4, 4>), grid, dim3(4 * 64), 0, s, ra);
        else hipLaunchKernelGGL((lp::dev::row_kernel<4, 2>), grid, dim3(4 * 64), 0, s, ra);
    }
    LP_HIP_TRY(hipGetLastError());
    if (plan->split > 1) {
        lp::dev::MergeArgs ma;
        ma.src = src;
        ma.vocab = plan->vocab;
        ma.split = plan->split;
        ma.out_rows = static_cast<uint32_t>(plan->out_rows);
        ma.desc = desc;
        ma.partials = partials;
        ma.out_lp = out_logprobs;
        ma.out_id = out_token_ids;
        const uint32_t mblocks = static_cast<uint32_t>((plan->out_rows + 3) / 4);
        hipLaunchKernelGGL(lp::dev::merge_kernel, dim3(mblocks), dim3(256), 0, s, ma);
        LP_HIP_TRY(hipGetLastError());
    }
    return LP_OK;
}

lp_status lp_compute_ragged(lp_plan *plan, const float *logits, const float *next_token_logits,
                            const uint32_t *tokens, const uint32_t *sampled_tokens,
                            float *out_logprobs, uint32_t *out_token_ids, void *workspace,
                            uint64_t workspace_bytes, void *stream) {
    lp_status st = lp_stage_ragged(plan, tokens, sampled_tokens, workspace, workspace_bytes, stream);
    if (st != LP_OK) return st;
    return lp_launch_ragged(plan, logits, next_token_logits, out_logprobs, out_token_ids,
                            workspace, workspace_bytes, stream);
}

lp_status lp_bench_stream_read(const float *x, uint64_t n, float *partial_out, uint32_t *grid_out,
                               void *stream) {
    if (x == nullptr || partial_out == nullptr || grid_out == nullptr) return LP_ERR_NULL_ARG;
    if ((reinterpret_cast<uintptr_t>(x) & 15u) != 0) return LP_ERR_UNSUPPORTED;
    const uint64_t n4 = n / 4;
    const uint32_t ntail = static_cast<uint32_t>(n - n4 * 4);
    uint64_t grid = n4 / (256ull * 16ull);
    if (grid < 1) grid = 1;
    if (grid > 65536) grid = 65536;
    *grid_out = static_cast<uint32_t>(grid);
    hipLaunchKernelGGL(lp::dev::stream_read_kernel, dim3(static_cast<uint32_t>(grid)), dim3(256), 0,
                       static_cast<hipStream_t>(stream), reinterpret_cast<const float4 *>(x), n4,
                       x + n4 * 4, ntail, partial_out);
    LP_HIP_TRY(hipGetLastError());
    return LP_OK;
}

}  // extern "C"
