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
//  * Each row (or row segment) is one workgroup of kWaves waves.  Waves take
//    interleaved chunks of 64 lanes x kU float4.  Per chunk a lane reduces its
//    16 values to a chunk max, updates a running (m, s) with s = sum e^(x-m)
//    (exp2 with log2(e) folded in after an exact subtraction), and compares
//    one order key -- built from the chunk max and the lane's first token id --
//    against the wave's threshold.
//  * Ranking uses a 64-bit order key: the fp32 bits mapped to an unsigned
//    order (with -0.0 folded onto +0.0) in the high word, the complemented
//    token id in the low word.  A larger key is a better (value, id) pair, so
//    ties go to the lowest id and every merge in the kernel uses one total
//    order.
//  * A wave keeps candidates (keys above its threshold T) in an LDS buffer.
//    When it fills, the wave selects its 7 best keys (7 rounds of a wave-wide
//    max) and raises T to the 7th.  Any T that 7 real keys reach is a valid
//    cut, so the first chunk seeds T from the 7th largest lane maximum and
//    waves of one workgroup share their T through LDS.  After the first chunk
//    only a handful of chunks per row take this slow path.
//  * The waves' (m, s) pairs and candidate lists merge through LDS; the
//    epilogue writes lp = x - (m + ln s) for the 7 slots and the chosen token.
//  * With too few rows to fill 256 CUs, a row is split into segments, one
//    workgroup each; segments write (m, s, 7 keys) records and a merge kernel
//    (one wave per row) combines them in a fixed order and runs the epilogue.
//
// No MFMA: there is no contraction here.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "lp_internal.h"

namespace lp {
namespace dev {

constexpr int kWave = 64;
constexpr int kWaves = 4;            // waves per workgroup
constexpr int kThreads = kWave * kWaves;
constexpr int kU = 4;                // float4 loads per lane per chunk
constexpr int kChunkF4 = kWave * kU; // float4 per wave-chunk
constexpr int kCap = 256;            // candidate keys per wave buffer
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

__device__ __forceinline__ uint64_t uniform64(uint64_t v) {
    const uint32_t lo = __builtin_amdgcn_readfirstlane(uint32_t(v));
    const uint32_t hi = __builtin_amdgcn_readfirstlane(uint32_t(v >> 32));
    return (uint64_t(hi) << 32) | lo;
}

__device__ __forceinline__ float wave_max_f32(float v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
    return v;
}

__device__ __forceinline__ uint64_t wave_max_u64(uint64_t k) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) k = umax64(k, __shfl_xor(k, o));
    return k;
}

__device__ __forceinline__ uint32_t lanes_below(uint64_t mask) {
    return __builtin_amdgcn_mbcnt_hi(uint32_t(mask >> 32),
                                     __builtin_amdgcn_mbcnt_lo(uint32_t(mask), 0u));
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// (m, s) with s = sum e^(x - m): merge (m2, s2) into (m, s).  A max of -inf
// (nothing finite seen) contributes nothing and never forms -inf - -inf.
__device__ __forceinline__ void lse_merge(float &m, float &s, float m2, float s2) {
    const float M = fmaxf(m, m2);
    const float Ms = (M == -INFINITY) ? 0.0f : M;
    s = s * fast_exp2((m - Ms) * kLog2e) + s2 * fast_exp2((m2 - Ms) * kLog2e);
    m = M;
}

__device__ __forceinline__ void wave_lse(float &m, float &s) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
        const float m2 = __shfl_xor(m, o);
        const float s2 = __shfl_xor(s, o);
        lse_merge(m, s, m2, s2);
    }
}

// Best 7 keys of up to kPer*64 keys held kPer per lane (0 = empty).  Returns,
// in lane r < 7, the r-th best key (0 if fewer exist); every lane gets the
// count of nonzero keys found in *count.
template <int kPer>
__device__ __forceinline__ uint64_t wave_select7(uint64_t (&e)[kPer], int lane, uint32_t *count) {
    uint64_t mine = 0;
    uint32_t found = 0;
#pragma unroll
    for (int r = 0; r < kSlots; ++r) {
        uint64_t b = e[0];
#pragma unroll
        for (int i = 1; i < kPer; ++i) b = umax64(b, e[i]);
        b = uniform64(wave_max_u64(b));
        if (b == 0) break;  // uniform: nothing left
#pragma unroll
        for (int i = 0; i < kPer; ++i) e[i] = (e[i] == b) ? 0ull : e[i];  // keys are unique
        if (lane == r) mine = b;
        ++found;
    }
    *count = found;
    return mine;
}

// ------------------------------------------------------------------ candidates

struct WaveCands {
    uint64_t *buf;  // this wave's kCap keys in LDS
    uint32_t n;     // keys held (wave-uniform)
    uint64_t T;     // keep only keys > T (wave-uniform)
};

// Keeps the 7 best keys at buf[0..7) and raises T to the 7th.
__device__ __forceinline__ void compress(WaveCands &c, int lane) {
    constexpr int kPer = kCap / kWave;
    uint64_t e[kPer];
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
        const uint32_t idx = uint32_t(lane + kWave * i);
        e[i] = idx < c.n ? c.buf[idx] : 0ull;
    }
    uint32_t found;
    const uint64_t mine = wave_select7<kPer>(e, lane, &found);
    if (lane < int(found)) c.buf[lane] = mine;
    c.n = found;
    if (found == uint32_t(kSlots)) {
        const uint64_t seventh = uniform64(__shfl(mine, kSlots - 1));
        c.T = umax64(c.T, seventh);
    }
}

// Appends the keys of lanes where `pred` holds.
__device__ __forceinline__ void push(WaveCands &c, uint64_t key, bool pred, int lane) {
    uint64_t mask = __ballot(pred);
    if (mask == 0) return;
    if (c.n + uint32_t(__popcll(mask)) > uint32_t(kCap)) {
        compress(c, lane);
        pred = pred && key > c.T;
        mask = __ballot(pred);
        if (mask == 0) return;
    }
    const uint32_t pos = c.n + lanes_below(mask);
    if (pred) c.buf[pos] = key;
    c.n += uint32_t(__popcll(mask));
}

// First full chunk of a wave: 7 distinct elements (the maxima of 7 lanes) are
// at least the 7th largest lane maximum t, so every key below (t, any id) can
// be dropped.  Sets T just under the smallest key of value t.
__device__ __forceinline__ void seed_threshold(WaveCands &c, float lane_max) {
    float v = lane_max;
    float t = -INFINITY;
    uint32_t cnt = 0;
#pragma unroll
    for (int r = 0; r < kSlots; ++r) {
        const float mx = wave_max_f32(v);
        const uint64_t eq = __ballot(v == mx);
        cnt += uint32_t(__popcll(eq));
        t = mx;
        if (cnt >= uint32_t(kSlots)) break;
        v = (v == mx) ? -INFINITY : v;
    }
    if (cnt >= uint32_t(kSlots)) {
        const uint64_t k = uniform64(order_key(t, kPadId));  // low word 0: smallest key of value t
        if (k > 0) c.T = umax64(c.T, k - 1);
    }
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
    uint32_t *out_id;
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

__global__ __launch_bounds__(kThreads) void row_kernel(RowArgs a) {
    __shared__ uint64_t s_buf[kWaves][kCap];
    __shared__ uint64_t s_T;
    __shared__ float s_m[kWaves], s_s[kWaves];
    __shared__ uint32_t s_n[kWaves];

    const int tid = int(threadIdx.x);
    const int lane = tid & (kWave - 1);
    const int wave = tid >> 6;
    const uint32_t o = blockIdx.x / a.split;
    const uint32_t seg = blockIdx.x - o * a.split;
    const RowDesc d = a.desc[o];

    if (d.top_n == 0) {  // padding-only row: no logits read
        if (a.split == 1 && wave == 0) write_padding(a.out_lp, a.out_id, o, lane);
        return;
    }

    const uint32_t V = a.vocab;
    const float *row = a.src + uint64_t(d.src_row) * V;
    const uint64_t seg_start = uint64_t(seg) * a.seg_len;
    const uint32_t v0 = seg_start < V ? uint32_t(seg_start) : V;
    const uint32_t v1 = (uint64_t(v0) + a.seg_len < V) ? v0 + a.seg_len : V;

    if (tid == 0) s_T = 0;
    __syncthreads();

    WaveCands c{s_buf[wave], 0u, 0ull};
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

    auto load_chunk = [&](float4 (&x)[kU], uint32_t ch) {
        const float4 *p = body + uint64_t(ch) * kChunkF4 + lane;
#pragma unroll
        for (int u = 0; u < kU; ++u) x[u] = p[u * kWave];
    };

    auto process_chunk = [&](const float4 (&x)[kU], uint32_t ch) {
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

        const uint32_t first_id = a0 + 4u * (ch * uint32_t(kChunkF4) + uint32_t(lane));
        const uint64_t kc = order_key(cm, first_id);
        if (__ballot(kc > c.T) == 0) return;              // common case
        c.T = umax64(c.T, uniform64(*(volatile uint64_t *)&s_T));
        if (__ballot(kc > c.T) == 0) return;
        const uint64_t t_before = c.T;
        if (c.T == 0) seed_threshold(c, cm);
#pragma unroll
        for (int u = 0; u < kU; ++u) {
            const uint32_t id = a0 + 4u * (ch * uint32_t(kChunkF4) + uint32_t(u * kWave + lane));
            const uint64_t k0 = order_key(x[u].x, id + 0);
            push(c, k0, k0 > c.T, lane);
            const uint64_t k1 = order_key(x[u].y, id + 1);
            push(c, k1, k1 > c.T, lane);
            const uint64_t k2 = order_key(x[u].z, id + 2);
            push(c, k2, k2 > c.T, lane);
            const uint64_t k3 = order_key(x[u].w, id + 3);
            push(c, k3, k3 > c.T, lane);
        }
        if (c.T != t_before && lane == 0) atomicMax((unsigned long long *)&s_T, c.T);
    };

    // two chunks in flight per wave
    {
        float4 xa[kU], xb[kU];
        uint32_t ch = uint32_t(wave);
        if (ch < nchunks) load_chunk(xa, ch);
        while (ch < nchunks) {
            const uint32_t ch2 = ch + kWaves;
            if (ch2 < nchunks) load_chunk(xb, ch2);
            process_chunk(xa, ch);
            ch = ch2;
            if (ch >= nchunks) break;
            const uint32_t ch3 = ch + kWaves;
            if (ch3 < nchunks) load_chunk(xa, ch3);
            process_chunk(xb, ch);
            ch = ch3;
        }
    }

    // head (before a0) and tail (after the last full chunk): one element per
    // thread per pass
    {
        c.T = umax64(c.T, uniform64(*(volatile uint64_t *)&s_T));
        const uint32_t nh = a0 - v0;
        const uint32_t tail0 = a0 + nchunks * uint32_t(kChunkF4) * 4u;
        const uint32_t nrest = nh + (v1 - tail0);
        for (uint32_t base = 0; base < nrest; base += kThreads) {
            const uint32_t r = base + uint32_t(tid);
            const bool valid = r < nrest;
            const uint32_t e = (r < nh) ? v0 + r : tail0 + (r - nh);
            const float x = valid ? row[e] : -INFINITY;
            const float mn = fmaxf(m, x);
            const float ms = (mn == -INFINITY) ? 0.0f : mn;
            s = s * fast_exp2((m - ms) * kLog2e) + fast_exp2((x - ms) * kLog2e);
            m = mn;
            const uint64_t k = valid ? order_key(x, e) : 0ull;
            push(c, k, valid && k > c.T, lane);
        }
    }

    // per wave: (m, s) across lanes, candidates down to <= 7
    wave_lse(m, s);
    if (c.n > uint32_t(kSlots)) compress(c, lane);
    if (lane == 0) {
        s_m[wave] = m;
        s_s[wave] = s;
        s_n[wave] = c.n;
    }
    __syncthreads();
    if (wave != 0) return;

    // workgroup merge in wave 0
    constexpr int kPer = (kWaves * kSlots + kWave - 1) / kWave;
    uint64_t e[kPer];
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
        const int idx = lane + kWave * i;
        const int w = idx / kSlots, j = idx - (idx / kSlots) * kSlots;
        e[i] = (w < kWaves && uint32_t(j) < s_n[w < kWaves ? w : 0]) ? s_buf[w < kWaves ? w : 0][j] : 0ull;
    }
    uint32_t found;
    const uint64_t mine = wave_select7<kPer>(e, lane, &found);
    float M = lane < kWaves ? s_m[lane < kWaves ? lane : 0] : -INFINITY;
    float S = lane < kWaves ? s_s[lane < kWaves ? lane : 0] : 0.0f;
    wave_lse(M, S);

    if (a.split == 1) {
        const float lse = M + logf(S);
        write_row(a.out_lp, a.out_id, o, lane, mine, d.top_n, lse, row, d.chosen);
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

// One wave per output row: combines the row's `split` segment records in
// segment order, then writes the row.
__global__ __launch_bounds__(kThreads) void merge_kernel(MergeArgs a) {
    const int lane = int(threadIdx.x) & (kWave - 1);
    const uint32_t o = blockIdx.x * kWaves + (threadIdx.x >> 6);
    if (o >= a.out_rows) return;
    const RowDesc d = a.desc[o];
    if (d.top_n == 0) {
        write_padding(a.out_lp, a.out_id, o, lane);
        return;
    }
    const PartialRec *recs = a.partials + uint64_t(o) * a.split;
    float M = -INFINITY, S = 0.0f;
    if (uint32_t(lane) < a.split) {
        M = recs[lane].m;
        S = recs[lane].s;
    }
    wave_lse(M, S);

    constexpr int kPer = (int(kMaxSplit) * kSlots + kWave - 1) / kWave;
    const uint32_t nkeys = a.split * uint32_t(kSlots);
    uint64_t e[kPer];
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
        const uint32_t idx = uint32_t(lane + kWave * i);
        e[i] = idx < nkeys ? recs[idx / kSlots].keys[idx % kSlots] : 0ull;
    }
    uint32_t found;
    const uint64_t mine = wave_select7<kPer>(e, lane, &found);
    const float *row = a.src + uint64_t(d.src_row) * a.vocab;
    const float lse = M + logf(S);
    write_row(a.out_lp, a.out_id, o, lane, mine, d.top_n, lse, row, d.chosen);
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
    const uint64_t blocks = plan->out_rows * plan->split;
    if (blocks * lp::dev::kThreads >= (1ull << 32)) return LP_ERR_UNSUPPORTED;

    hipStream_t s = static_cast<hipStream_t>(stream);
    auto *desc = static_cast<const lp::RowDesc *>(workspace);
    auto *partials = reinterpret_cast<lp::PartialRec *>(static_cast<char *>(workspace) +
                                                        plan->desc_bytes);
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
    hipLaunchKernelGGL(lp::dev::row_kernel, dim3(static_cast<uint32_t>(blocks)),
                       dim3(lp::dev::kThreads), 0, s, ra);
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
        const uint32_t mblocks =
            static_cast<uint32_t>((plan->out_rows + lp::dev::kWaves - 1) / lp::dev::kWaves);
        hipLaunchKernelGGL(lp::dev::merge_kernel, dim3(mblocks), dim3(lp::dev::kThreads), 0, s,
                           ma);
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
