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
//    loads.  Per chunk a lane
//    reduces its 16 values to a chunk max, updates a running (m, s) with
//    s = sum e^(x-m) (exp2 with log2(e) applied after an exact subtraction),
//    and compares one order key -- built from the chunk max and the lane's
//    first token id -- against the wave's threshold T.
//  * Ranking uses a 64-bit order key: the fp32 bits mapped to an unsigned
//    order (with -0.0 folded onto +0.0) in the high word, the complemented
//    token id in the low word.  A larger key is a better (value, id) pair, so
//    ties go to the lowest id and every merge uses one total order.
//  * Each wave keeps its exact top-7 keys so far spread over lanes 0..6, and
//    T = the 7th of them, raised further to any T another wave of the
//    workgroup has published in LDS (a key that 7 real elements beat can
//    never enter).  A chunk that beats T has its keys merged into the list:
//    one by one (a lane-parallel shift) when they are few, else by one
//    wave-wide selection over the chunk and the list.
//  * The waves' (m, s) pairs and top-7 lists merge through LDS; the
//    epilogue writes lp = x - (m + ln s) for the 7 slots and the chosen token.
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

__device__ __forceinline__ uint32_t wave_sum_u32(uint32_t v) {
    v += dpp_u32<kDppXor1>(v);
    v += dpp_u32<kDppXor2>(v);
    v += dpp_u32<kDppHalfMirror>(v);
    v += dpp_u32<kDppMirror>(v);
    return (readlane_u32(v, 0) + readlane_u32(v, 16)) + (readlane_u32(v, 32) + readlane_u32(v, 48));
}

__device__ __forceinline__ uint32_t lanes_below(uint64_t mask) {
    return __builtin_amdgcn_mbcnt_hi(uint32_t(mask >> 32),
                                     __builtin_amdgcn_mbcnt_lo(uint32_t(mask), 0u));
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Orders this wave's LDS accesses around an LDS counter: the workgroup-scope
// fences restricted to LDS wait only for outstanding LDS operations, never
// for the wave's in-flight global loads.
__device__ __forceinline__ void lds_release() { __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local"); }
__device__ __forceinline__ void lds_acquire() { __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local"); }

// Lane 0 adds 1 to an LDS counter; every lane gets the previous value.
__device__ __forceinline__ uint32_t lds_arrive(uint32_t *counter, int lane) {
    uint32_t prev = 0;
    if (lane == 0) prev = __hip_atomic_fetch_add(counter, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
    return readlane_u32(prev, 0);
}

// Logits are read exactly once: nontemporal 16-byte loads (the `nt` form of
// global_load_dwordx4) stream them without displacing reusable cache lines;
// on gfx950 they sustain ~13% more HBM bandwidth than plain loads here.
typedef float f32x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ float4 stream_load(const float4 *p) {
    const f32x4 v = __builtin_nontemporal_load(reinterpret_cast<const f32x4 *>(p));
    return make_float4(v.x, v.y, v.z, v.w);
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

constexpr int kInsertMax = 24;       // above this many candidates in a chunk, merge in bulk
constexpr int kDppShr1 = 0x111;      // row_shr:1: lane i reads lane i-1 of its row of 16

template <int kCtrl>
__device__ __forceinline__ uint64_t dpp_u64_or0(uint64_t v) {
    return (uint64_t(dpp_u32<kCtrl>(uint32_t(v >> 32))) << 32) | dpp_u32<kCtrl>(uint32_t(v));
}

// A wave's exact top-7 keys so far, spread over lanes: lane r < 7 holds the
// r-th best (0 = empty), other lanes hold 0.  T (wave-uniform) is the 7th
// key, or a larger bound that another wave of the workgroup published.
struct WaveTop {
    uint64_t L;
    uint64_t T;
};

// Inserts a wave-uniform key that is not in the list yet, all slots at once:
// slots holding smaller keys shift down by one lane (row_shr:1) and the first
// of them takes k.
__device__ __forceinline__ void top_insert(WaveTop &w, uint64_t k, int lane) {
    const uint64_t prev = dpp_u64_or0<kDppShr1>(w.L);   // slot above (lane 0: none)
    const bool below = k > w.L;
    const bool take_k = lane == 0 || prev > k;
    const uint64_t nl = below ? (take_k ? k : prev) : w.L;
    w.L = lane < kSlots ? nl : 0ull;
    w.T = umax64(w.T, readlane_u64(w.L, kSlots - 1));
}

// The smallest value a key above T can have; a cheap superset test for
// candidates (below the key of -inf, nothing is excluded).
__device__ __forceinline__ float threshold_value(uint64_t T) {
    return uint32_t(T >> 32) >= 0x007FFFFFu ? key_value(T) : -INFINITY;
}

// Exact merge of candidate keys (those above T) into the list by one
// wave-wide selection over the candidates and the list together.  A key
// already in the list may also be among the candidates: the selection removes
// every copy of the key it picks, so duplicates count once.
template <int kN>
__device__ __forceinline__ void bulk_merge(WaveTop &w, uint64_t (&f)[kN + 1], int lane) {
#pragma unroll
    for (int j = 0; j < kN; ++j) f[j] = f[j] > w.T ? f[j] : 0ull;
    f[kN] = w.L;
    uint32_t found;
    w.L = wave_select7<kN + 1>(f, lane, &found);
    w.T = umax64(w.T, readlane_u64(w.L, kSlots - 1));
}

// Inserts the keys of one column (one key per lane) that are above T.
// Returns false, inserting nothing, when that would exceed the budget.
__device__ __forceinline__ bool insert_column(WaveTop &w, uint64_t k, uint32_t &budget, int lane) {
    uint64_t mask = __ballot(k > w.T);
    if (mask == 0) return true;
    const uint32_t n = uint32_t(__popcll(mask));
    if (n > budget) return false;
    budget -= n;
    while (mask != 0) {
        const int l = __builtin_ctzll(mask);
        mask &= mask - 1;
        top_insert(w, readlane_u64(k, l), lane);
    }
    return true;
}

__device__ __forceinline__ float f4_get(const float4 &v, int q) {
    return q == 0 ? v.x : q == 1 ? v.y : q == 2 ? v.z : v.w;
}

// Raises T from the lanes' running maxima: if 7 lanes have each seen an
// element of value >= t (counting lanes that tie), no element below t can be
// in the top 7, so T may rise to just under the smallest key of value t.
// Every lane's running max must be a real element of this wave's range.
__device__ __forceinline__ void tighten_from_lane_max(WaveTop &w, float lane_max) {
    float v = lane_max;
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
    if (cnt >= uint32_t(kSlots)) {
        const uint64_t k = order_key(t, kPadId);  // low word 0: smallest key of value t
        if (k > 0) w.T = umax64(w.T, k - 1);
    }
}

// Seeds T from the first-chunk maxima of all waves of the workgroup
// (vals: kN values per lane, -inf where a wave had no chunk): the 7th largest,
// counting ties, is reached by 7 distinct real elements unless it is -inf,
// and a -inf bound excludes nothing.  Every wave computes the same T.
template <int kN>
__device__ __forceinline__ void seed_from_maxima(WaveTop &w, float (&v)[kN]) {
    float t = -INFINITY;
    uint32_t cnt = 0;
#pragma unroll 1
    for (int r = 0; r < kSlots; ++r) {
        float lm = v[0];
#pragma unroll
        for (int i = 1; i < kN; ++i) lm = fmaxf(lm, v[i]);
        const float mx = wave_max_f32(lm);
        uint32_t c = 0;
#pragma unroll
        for (int i = 0; i < kN; ++i) c += v[i] == mx ? 1u : 0u;
        cnt += wave_sum_u32(c);
        t = mx;
        if (cnt >= uint32_t(kSlots)) break;
#pragma unroll
        for (int i = 0; i < kN; ++i) v[i] = v[i] == mx ? -INFINITY : v[i];
    }
    if (cnt >= uint32_t(kSlots)) {
        const uint64_t k = order_key(t, kPadId);
        if (k > 0) w.T = umax64(w.T, k - 1);
    }
}

// Merges a chunk's keys above T into the list.  A wave whose T is still 0
// first seeds it from its own lanes' maxima.  A float compare against T's value skips
// the columns with no candidate; the others are inserted while few
// candidates arrive, else (heavy ties) the chunk is merged in bulk, one
// float4 column group at a time.  Keys are rebuilt in the bulk path from
// register copies the compiler cannot see through, so the common path never
// keeps a chunk's keys alive.
template <int kU_>
__device__ __forceinline__ void chunk_merge(WaveTop &w, const float4 (&x)[kU_], uint32_t first_id,
                                            float lane_max, int lane) {
    if (w.T == 0) tighten_from_lane_max(w, lane_max);
    uint32_t budget = uint32_t(kInsertMax);
    const float tv = threshold_value(w.T);
    bool ok = true;
#pragma unroll
    for (int j = 0; j < 4 * kU_; ++j) {
        const int u = j >> 2, q = j & 3;
        const float v = f4_get(x[u], q);
        if (__ballot(v >= tv) == 0) continue;
        const uint64_t k = order_key(v, first_id + 4u * uint32_t(u * kWave) + q);
        if (!insert_column(w, k, budget, lane)) {
            ok = false;
            break;
        }
    }
    if (ok) return;
#pragma unroll
    for (int u = 0; u < kU_; ++u) {
        float y[4] = {x[u].x, x[u].y, x[u].z, x[u].w};
#pragma unroll
        for (int q = 0; q < 4; ++q) asm volatile("" : "+v"(y[q]));
        const uint32_t id = first_id + 4u * uint32_t(u * kWave);
        uint64_t f[5];
#pragma unroll
        for (int q = 0; q < 4; ++q) f[q] = order_key(y[q], id + uint32_t(q));
        bulk_merge<4>(w, f, lane);
    }
}

// One key per lane (head / tail elements).
__device__ __forceinline__ void single_merge(WaveTop &w, uint64_t k, int lane) {
    uint32_t budget = uint32_t(kInsertMax);
    if (insert_column(w, k, budget, lane)) return;
    uint64_t f[2] = {k, 0ull};
    bulk_merge<1>(w, f, lane);
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
                                          const float *row, uint32_t chosen) {
    // lanes 0..6: ranked slots; lane 7: the chosen token
    if (lane < kSlots) {
        const bool valid = uint32_t(lane) < top_n && key != 0;
        out_lp[o * kCols + lane] = valid ? key_value(key) - lse : -INFINITY;
        out_id[o * kCols + lane] = valid ? key_id(key) : kPadId;
    } else if (lane == kSlots) {
        out_lp[o * kCols + lane] = row[chosen] - lse;
        out_id[o * kCols + lane] = chosen;
    }
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
    __shared__ uint64_t s_keys[kWaves * kSlots];
    __shared__ float s_lmax[kWaves * kWave];
    __shared__ uint64_t s_T;
    __shared__ float s_m[kWaves], s_s[kWaves];
    __shared__ uint32_t s_seeded, s_done;

    const int tid = int(threadIdx.x);
    const int lane = tid & (kWave - 1);
    const int wave = tid >> 6;
    const uint32_t o = blockIdx.x / a.split;
    const uint32_t seg = blockIdx.x - o * a.split;
    const RowDesc d = a.desc[o];

    if (d.top_n == 0) {  // padding-only row: no logits read (the merge kernel pads split rows)
        if (a.split == 1 && wave == 0) write_padding(a.out_lp, a.out_id, o, lane);
        return;
    }

    const uint32_t V = a.vocab;
    const float *row = a.src + uint64_t(d.src_row) * V;
    const uint64_t seg_start = uint64_t(seg) * a.seg_len;
    const uint32_t v0 = seg_start < V ? uint32_t(seg_start) : V;
    const uint32_t v1 = (uint64_t(v0) + a.seg_len < V) ? v0 + a.seg_len : V;

    WaveTop w{0ull, 0ull};
    float m = -INFINITY, s = 0.0f;

    // aligned body: float4 loads from a 16-byte aligned element a0
    uint32_t a0 = v0;
    {
        const uint32_t mis = uint32_t((reinterpret_cast<uintptr_t>(row + v0) >> 2) & 3u);
        a0 = v0 + ((4u - mis) & 3u);
        if (a0 > v1) a0 = v1;
    }
    const uint32_t nf4 = (v1 - a0) >> 2;
    const uint32_t nchunks = nf4 / uint32_t(kChunkF4);
    const float4 *body = reinterpret_cast<const float4 *>(row + a0);

    auto load_chunk = [&](float4 (&x)[kU], uint32_t ch) __attribute__((always_inline)) {
        const float4 *p = body + uint64_t(ch) * kChunkF4 + lane;
#pragma unroll
        for (int u = 0; u < kU; ++u) x[u] = stream_load(p + u * kWave);
    };

    // LSE update for one chunk; returns the lane's chunk max
    auto lse_chunk = [&](const float4 (&x)[kU]) __attribute__((always_inline)) {
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

    // top-k part for one chunk whose lane maxima are cm
    auto topk_chunk = [&](const float4 (&x)[kU], uint32_t ch, float cm) __attribute__((always_inline)) {
        // any element of this lane's chunk has a key <= order_key(cm, first_id)
        const uint32_t first_id = a0 + 4u * (ch * uint32_t(kChunkF4) + uint32_t(lane));
        const uint64_t kc = order_key(cm, first_id);
        if (__ballot(kc > w.T) == 0) return;              // common case
        const uint64_t t_before = w.T;
        w.T = umax64(w.T, uniform64(*(volatile uint64_t *)&s_T));
        if (__ballot(kc > w.T) == 0) return;
        chunk_merge<kU>(w, x, first_id, m, lane);
        if (w.T != t_before && lane == 0) atomicMax((unsigned long long *)&s_T, w.T);
    };

    auto process_chunk = [&](const float4 (&x)[kU], uint32_t ch) __attribute__((always_inline)) {
        const float cm = lse_chunk(x);
        topk_chunk(x, ch, cm);
    };

    // kDepth chunks in flight per wave (register buffers used in rotation).
    // Each wave publishes its first chunk's lane maxima; the last wave to do
    // so seeds one threshold for the whole workgroup from all of them, while
    // the others carry on (no wave waits for another).
    {
        float4 xb[kDepth][kU];
        uint32_t ch = uint32_t(wave);
#pragma unroll
        for (int d = 0; d < kDepth; ++d)
            if (ch + uint32_t(d * kWaves) < nchunks) load_chunk(xb[d], ch + uint32_t(d * kWaves));
        if (tid == 0) {
            s_T = 0;
            s_seeded = 0;
            s_done = 0;
        }
        __syncthreads();
        float cm0 = -INFINITY;
        if (ch < nchunks) cm0 = lse_chunk(xb[0]);
        s_lmax[wave * kWave + lane] = cm0;
        lds_release();
        if (lds_arrive(&s_seeded, lane) == uint32_t(kWaves - 1)) {
            lds_acquire();
            float v[kWaves];
#pragma unroll
            for (int i = 0; i < kWaves; ++i) v[i] = s_lmax[i * kWave + lane];
            seed_from_maxima<kWaves>(w, v);
            if (lane == 0) atomicMax((unsigned long long *)&s_T, w.T);
        }
        if (ch < nchunks) topk_chunk(xb[0], ch, cm0);
        constexpr uint32_t kAhead = uint32_t(kDepth * kWaves);
        if (ch + kAhead < nchunks) load_chunk(xb[0], ch + kAhead);
        ch += kWaves;
        // buffer d % kDepth holds chunk ch on the d-th step of each round
        while (ch < nchunks) {
#pragma unroll
            for (int d = 1; d <= kDepth; ++d) {
                if (ch >= nchunks) break;
                process_chunk(xb[d % kDepth], ch);
                if (ch + kAhead < nchunks) load_chunk(xb[d % kDepth], ch + kAhead);
                ch += kWaves;
            }
        }
    }

    // head (before a0) and tail (after the last full chunk): one element per
    // thread per pass
    {
        w.T = umax64(w.T, uniform64(*(volatile uint64_t *)&s_T));
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
            single_merge(w, valid ? order_key(x, e) : 0ull, lane);
        }
    }

    // per wave: (m, s) across lanes and the wave's 7 keys into LDS; the last
    // wave of the workgroup to get here merges them
    wave_lse(m, s);
    if (lane < kSlots) s_keys[wave * kSlots + lane] = w.L;
    if (lane == 0) {
        s_m[wave] = m;
        s_s[wave] = s;
    }
    lds_release();
    if (lds_arrive(&s_done, lane) != uint32_t(kWaves - 1)) return;
    lds_acquire();

    // workgroup merge: the kWaves * 7 keys spread over the lanes
    constexpr int kPer = (kWaves * kSlots + kWave - 1) / kWave;
    uint64_t e[kPer];
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
        const int idx = lane + kWave * i;
        e[i] = idx < kWaves * kSlots ? s_keys[idx < kWaves * kSlots ? idx : 0] : 0ull;
    }
    uint32_t found;
    const uint64_t mine = wave_select7<kPer>(e, lane, &found);
    float M = -INFINITY, S = 0.0f;
    if (lane < kWaves) {
        M = s_m[lane];
        S = s_s[lane];
    }
    wave_lse(M, S);

    if (a.split == 1) {
        write_row(a.out_lp, a.out_id, o, lane, mine, d.top_n, M + logf(S), row, d.chosen);
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
    const float *row = a.src + uint64_t(d.src_row) * a.vocab;
    write_row(a.out_lp, a.out_id, o, lane, top, d.top_n, m + logf(s), row, d.chosen);
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
    ra.seg_len = static_cast<uint32_t>(
        lp::align_up((uint64_t(plan->vocab) + plan->split - 1) / plan->split, 4));
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
