// topm.hip -- top-M marginal candidates per (request, block position) row.
//
// The builder precomputes the top-M marginal tokens of every depth before the
// expansion ([captcha] "Methodology -- deep read"; [gist] "Composants clés --
// Restriction de candidats (Top-M)").  Order: value desc, token id asc.
//
// The select is HBM-bound: every row of V logits is streamed once, in
// `nseg` segments of one 256-thread workgroup each, through buffer loads
// software-pipelined over two register sets (one batch in flight while the
// previous one is evaluated).  Every wave keeps the 64 best (value, ~id) keys
// it has admitted, sorted across its lanes, and an admission threshold: a key
// below it cannot be among the segment's 64 best.  Valid thresholds come from
//   (a) the 64th largest of the 256 lane maxima of the first batch (64
//       distinct elements reach it);
//   (b) the wave's own 64th best key;
//   (c) bounds the four waves share in LDS: the largest 64th best of any wave,
//       and the smallest of the four waves' 16th best keys (together the
//       waves hold 64 keys at or above it).
// The hot loop is one conservative max-reduction and one compare per 16-byte
// vector; a vector whose maximum reaches the threshold is stashed in LDS, and
// stashed vectors are evaluated 64 at a time (one per lane), which amortizes
// the wave-wide work of admitting a key.  Admitted keys are folded into the
// list by insertion (few keys) or bitonic sort + merge.  With several segments
// per row, topm_merge folds a row's partial lists into its top M.
//
// Full-vocabulary mode (TAIL): the same pass also sums exp(x / T) (T = 1 when
// T = 0) over the row's logits outside its top M, the tail that the
// full-vocabulary softmax adds to a node's normalizer.  Every element of the
// row is counted exactly once: those of vectors the filter rejects, stashed
// elements below the threshold, admitted keys that later drop out of a list
// (insertion, merge), keys that lose the final merges, and list entries past
// M.  Per lane the sum is held as s * 2^m with y = x * log2(e) / T; elements
// of rejected vectors lie below the threshold, so with m kept at least the
// threshold they add 2^(y - m) <= 1 without a compare.
#include <cfloat>

#include "dt_device.h"
#include "dt_launch.h"

namespace dt {

namespace {

constexpr int kTopmThreads = 256;
constexpr int kWaves = kTopmThreads / kWave;
constexpr int kUnroll = 4;  // 16-byte vectors per lane per batch (two batches in flight)
// stashed vectors per wave: fewer than 64 left over plus at most 64 per vector of a batch
constexpr int kStash = kWave * (kUnroll + 1);

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

template <typename T> struct Elem;
template <> struct Elem<float> {
    static constexpr int kPerVec = 4;
    __device__ static float get(const u32x4& v, int i) {
        return __uint_as_float(i == 0 ? v.x : i == 1 ? v.y : i == 2 ? v.z : v.w);
    }
    __device__ static float vmax(const u32x4& v) {
        return fmaxf(fmaxf(__uint_as_float(v.x), __uint_as_float(v.y)),
                     fmaxf(__uint_as_float(v.z), __uint_as_float(v.w)));
    }
    // binary32 elements are compared exactly
    static constexpr float kSlack = 0.f;
    __device__ static float vfilter(const u32x4& v) { return vmax(v); }
    __device__ static float scalar(const float* p) { return *p; }
};
template <> struct Elem<bf16_t> {
    static constexpr int kPerVec = 8;
    __device__ static float get(const u32x4& v, int i) {
        const uint32_t x = (i >> 1) == 0 ? v.x : (i >> 1) == 1 ? v.y : (i >> 1) == 2 ? v.z : v.w;
        return __uint_as_float((i & 1) ? (x & 0xFFFF0000u) : (x << 16));
    }
    __device__ static float vmax(const u32x4& v) {
        float a = fmaxf(__uint_as_float(v.x << 16), __uint_as_float(v.x & 0xFFFF0000u));
        float b = fmaxf(__uint_as_float(v.y << 16), __uint_as_float(v.y & 0xFFFF0000u));
        float c = fmaxf(__uint_as_float(v.z << 16), __uint_as_float(v.z & 0xFFFF0000u));
        float d = fmaxf(__uint_as_float(v.w << 16), __uint_as_float(v.w & 0xFFFF0000u));
        return fmaxf(fmaxf(a, b), fmaxf(c, d));
    }
    // An upper bound on the element maximum within |value| / 128 of it, in 8
    // operations instead of 12: a 32-bit word read as binary32 is its high
    // bf16 element plus part of the low one's bits, i.e. the high element
    // moved away from zero by less than 2^-7 of its magnitude, or, when the
    // high element is a zero or a denormal, by less than 2^-133 (a -0.0 high
    // element then reads as a negative denormal).  Vectors are therefore
    // compared with a threshold lowered by |threshold| / 64 + FLT_MIN, which
    // never rejects an element at or above the threshold.
    static constexpr float kSlack = 1.f / 64.f;
    __device__ static float vfilter(const u32x4& v) {
        const float a = fmaxf(fmaxf(__uint_as_float(v.x), __uint_as_float(v.y)), __uint_as_float(v.z));
        const float b = fmaxf(fmaxf(__uint_as_float(v.w), __uint_as_float(v.x << 16)),
                              __uint_as_float(v.y << 16));
        const float c = fmaxf(fmaxf(__uint_as_float(v.z << 16), __uint_as_float(v.w << 16)), a);
        return fmaxf(b, c);
    }
    __device__ static float scalar(const bf16_t* p) { return bf16_to_f32(*p); }
};

// Per-wave running top-64: `list` (one key per lane, descending), a staging
// buffer of admitted keys in LDS and the admission threshold `thr` (keys
// below it are rejected; 0 admits everything).
struct WaveTop {
    u64 list;
    u64 thr;
    float thr_val;  // value part of thr (-inf while thr == 0)
    float filt;     // vector filter bound: thr_val lowered by slack * |thr_val| (bf16: and FLT_MIN), >= -FLT_MAX
    float slack;
    int nbuf;
};

// Per-lane tail sum: sum of 2^(y - m) over the values added, y = x * c.
struct TailAcc {
    float m;  // -FLT_MAX while empty (2^(y - m) of any finite y is then 0)
    float s;
    float c;  // log2(e) / T
};
__device__ __forceinline__ void tail_add(TailAcc& t, float x) {  // any value
    const float y = x * t.c;
    if (y > t.m) {
        t.s = t.s * __builtin_amdgcn_exp2f(t.m - y) + 1.f;
        t.m = y;
    } else {
        t.s += __builtin_amdgcn_exp2f(y - t.m);
    }
}
// x * c <= m: no compare
__device__ __forceinline__ void tail_add_below(TailAcc& t, float x) {
    t.s += __builtin_amdgcn_exp2f(fmaf(x, t.c, -t.m));
}
// Keep m at or above the threshold's y (raised 8 above it, so that it moves
// only when the threshold has risen by 8 since).
__device__ __forceinline__ void tail_cover(TailAcc& t, float thr_val) {
    const float ty = thr_val * t.c;
    if (ty > t.m) {
        const float nm = ty + 8.f;
        t.s *= __builtin_amdgcn_exp2f(t.m - nm);
        t.m = nm;
    }
}
// (m, s) of a whole wave: the largest m and the rescaled sum (wave-uniform)
__device__ __forceinline__ void tail_wave_total(const TailAcc& t, float& M, float& S) {
    M = wave_max(t.m);
    S = wave_sum(t.s * __builtin_amdgcn_exp2f(t.m - M));
}
__device__ __forceinline__ void tail_join(float& M, float& S, float m2, float s2) {
    const float nm = fmaxf(M, m2);
    S = S * __builtin_amdgcn_exp2f(M - nm) + s2 * __builtin_amdgcn_exp2f(m2 - nm);
    M = nm;
}
// natural log of the tail, sum of exp(x / T) = 2^M * S; -inf when nothing was added
__device__ __forceinline__ float tail_lse(float M, float S) {
    return S > 0.f ? (M + __log2f(S)) * 0.6931471805599453f : -INFINITY;
}

__device__ __forceinline__ void set_thr(WaveTop& w, u64 t) {
    if (t > w.thr) {
        w.thr = t;
        w.thr_val = topm_key_val(t);
        // finite, so that masked vectors (-inf) never pass; the bf16 slack
        // also covers zero and denormal high elements (FLT_MIN)
        w.filt = fmaxf(w.slack > 0.f ? w.thr_val - fabsf(w.thr_val) * w.slack - FLT_MIN : w.thr_val, -FLT_MAX);
    }
}

// Value bounds the waves of a workgroup share (order-preserving value bits,
// 0 = none yet).  Both only rise.
//   max64:  the largest 64th-best value of any wave's list;
//   q16[w]: the 16th-best value of wave w's list.
// Wave lists only improve, so wave w keeps holding 16 keys >= q16[w]: the four
// waves together hold 64 keys >= min_w q16[w], and a key below that bound is
// not among the workgroup's 64 best.  With each wave seeing a quarter of the
// segment, this bound tracks the segment's own 64th best.
struct SharedThr {
    uint32_t max64;
    uint32_t q16[kWaves];
};

__device__ __forceinline__ u64 shared_bound(const SharedThr* st) {
    uint32_t q = __hip_atomic_load(&st->q16[0], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
#pragma unroll
    for (int i = 1; i < kWaves; ++i)
        q = min(q, __hip_atomic_load(&st->q16[i], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP));
    const uint32_t m = __hip_atomic_load(&st->max64, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
    return (u64)max(q, m) << 32;
}

// Publish the wave's bounds to the workgroup.
__device__ __forceinline__ void publish(const WaveTop& w, SharedThr* st) {
    const uint32_t q = (uint32_t)(bcast_u64(w.list, 15) >> 32);
    if (lane_id() == 0) {
        if (w.thr) atomicMax(&st->max64, (uint32_t)(w.thr >> 32));
        if (q) __hip_atomic_store(&st->q16[threadIdx.x / kWave], q, __ATOMIC_RELAXED,
                                  __HIP_MEMORY_SCOPE_WORKGROUP);
    }
}

// Folds of at most this many keys insert them one at a time (a ballot and a
// one-lane shift each); larger ones sort the buffer and merge it.
constexpr int kInsertMax = 16;

template <bool TAIL>
__device__ __forceinline__ void fold_buffer(WaveTop& w, TailAcc& ta, u64* buf, SharedThr* st) {
    const int lane = lane_id();
    if (w.nbuf <= kInsertMax) {
        for (int i = 0; i < w.nbuf; ++i) {
            const u64 k = buf[i];
            // the list is descending and its keys differ from k (ids differ)
            const int pos = __popcll(__ballot(w.list > k));
            if (pos >= kWave) {
                if (TAIL && lane == 0) tail_add(ta, topm_key_val(k));  // k drops out at once
                continue;
            }
            if (TAIL && lane == kWave - 1 && w.list) tail_add(ta, topm_key_val(w.list));  // shifted out
            const u64 sh = wave_shr1_u64(w.list);
            w.list = lane < pos ? w.list : (lane == pos ? k : sh);
        }
    } else {
        u64 x = lane < w.nbuf ? buf[lane] : 0ull;
        x = wave_sort(x, /*ascending=*/true);
        if (TAIL) {  // the 64 smaller of the 128 keys drop out
            const u64 lost = umin64(w.list, x);
            if (lost) tail_add(ta, topm_key_val(lost));
        }
        w.list = wave_merge_top64(w.list, x);
    }
    w.nbuf = 0;
    set_thr(w, bcast_u64(w.list, kWave - 1));
    publish(w, st);
    set_thr(w, shared_bound(st));
    if (TAIL) tail_cover(ta, w.thr_val);
}

// Offer one key per lane (valid only where `ok`); wave-uniform call.
template <bool TAIL>
__device__ __forceinline__ void offer(WaveTop& w, TailAcc& ta, u64* buf, SharedThr* s_thr, bool ok, u64 key) {
    bool pass = ok && key >= w.thr;
    u64 m = __ballot(pass);
    if (m == 0) {
        if (TAIL && ok) tail_add(ta, topm_key_val(key));
        return;
    }
    int cnt = __popcll(m);
    if (w.nbuf + cnt > kWave) {
        fold_buffer<TAIL>(w, ta, buf, s_thr);
        pass = ok && key >= w.thr;
        m = __ballot(pass);
        cnt = __popcll(m);
    }
    if (TAIL && ok && !pass) tail_add(ta, topm_key_val(key));
    if (pass) {
        const int pos = w.nbuf + (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32),
                                                                __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
        buf[pos] = key;
    }
    w.nbuf += cnt;
}

__device__ __forceinline__ int prefix_count(u64 m) {
    return (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
}

// Evaluate the last min(nst, 64) stashed vectors (one per lane) element by
// element.  The order in which admitted keys arrive does not change the
// result.  One copy of this code serves the whole kernel (its element loop is
// not unrolled), which keeps the kernel small enough for the instruction cache.
template <typename T, bool TAIL>
__device__ __forceinline__ void drain_stash(WaveTop& w, TailAcc& ta, u64* buf, SharedThr* s_thr,
                                            const u32x4* svec, const int* sidx, int& nst, int lo) {
    constexpr int P = Elem<T>::kPerVec;
    const int lane = lane_id();
    const int take = min(nst, kWave);
    const int from = nst - take;
    const bool on = lane < take;
    const u32x4 v = on ? svec[from + lane] : u32x4{0u, 0u, 0u, 0u};
    const int vi = on ? sidx[from + lane] : 0;
    set_thr(w, shared_bound(s_thr));
    // Elements at or above the bound as it stands (the others are out); a
    // vector passed the filter through one or two of them, so the offers
    // below take each lane's next pending element, lowest position first,
    // for as many rounds as the fullest lane needs instead of P.
    uint32_t pend = 0u;
#pragma unroll
    for (int i = 0; i < P; ++i) {
        const float x = Elem<T>::get(v, i);
        if (on && x >= w.thr_val) pend |= 1u << i;
        else if (TAIL && on) tail_add(ta, x);
    }
#pragma unroll 1
    while (__ballot(pend != 0u)) {
        const bool has = pend != 0u;
        const int i = has ? __builtin_ctz(pend) : 0;
        pend &= pend - 1u;
        offer<TAIL>(w, ta, buf, s_thr, has, topm_key(Elem<T>::get(v, i), (uint32_t)(lo + vi * P + i)));
    }
    // fold now, so that the shared bounds follow every admitted key
    if (w.nbuf) fold_buffer<TAIL>(w, ta, buf, s_thr);
    nst = from;
}

// With one segment per row the workgroup's list is the row's: it then writes
// the top M (idx, val) directly (and with TAIL the row's tail_lse to
// tail_out[row]) and no merge kernel runs; with several, each segment leaves
// its list in `partial` (and its tail sum (m, s), list excluded, in
// tail_part[row * nseg + segment]).  Workgroup (0, 0) also does the side job
// (TopmSide: a run of words zeroed, a clock pair set).
template <typename T, bool kVec, bool TAIL>
__global__ __launch_bounds__(kTopmThreads) void topm_partial_kernel(const T* __restrict__ base, int V,
                                                                    int nseg, int seg,
                                                                    u64* __restrict__ partial, int M,
                                                                    int32_t* __restrict__ idx,
                                                                    float* __restrict__ val, float tail_c,
                                                                    float* __restrict__ tail_out,
                                                                    float2* __restrict__ tail_part,
                                                                    TopmSide side) {
    __shared__ u64 sbuf[kWaves][kWave];
    __shared__ u32x4 svec[kWaves][kStash];
    __shared__ int sidx[kWaves][kStash];
    __shared__ SharedThr s_thr;
    __shared__ float2 s_tail[kWaves];
    const int row = blockIdx.x, s = blockIdx.y;  // rows along x: B * L is not limited to 16 bits
    const int wave = threadIdx.x / kWave, lane = lane_id();
    const T* rp = base + (size_t)row * (size_t)V;
    const int lo = s * seg;
    const int hi = min(V, lo + seg);
    u64* buf = sbuf[wave];
    if (threadIdx.x == 0) s_thr.max64 = 0u;
    if (threadIdx.x < kWaves) s_thr.q16[threadIdx.x] = 0u;
    if (row == 0 && s == 0) {  // the side job (see TopmSide)
        for (int i = threadIdx.x; i < side.nzero; i += kTopmThreads) side.zero[i] = 0u;
        if (side.clock && threadIdx.x < 2) side.clock[threadIdx.x] = threadIdx.x ? 0ull : ~0ull;
    }
    __syncthreads();

    WaveTop w;
    w.list = 0ull;
    w.thr = 0ull;
    w.thr_val = -INFINITY;
    w.filt = -FLT_MAX;
    w.slack = Elem<T>::kSlack;
    w.nbuf = 0;
    int nst = 0;
    TailAcc ta{-FLT_MAX, 0.f, tail_c};

    int tail_lo = lo;
    if (kVec && hi > lo) {
        constexpr int P = Elem<T>::kPerVec;
        constexpr int kBatch = kUnroll * kTopmThreads;
        const int nvec = (hi - lo) / P;
        // Buffer loads over the segment's whole vectors: reads past its end
        // return zeros (masked below), so the loop needs no address clamps.
        // The logits are read once: the loads are non-temporal (cache policy
        // bit 1), which keeps them from evicting, and writing back, what the
        // memory-side cache holds.
        const __amdgpu_buffer_rsrc_t rsrc =
            __builtin_amdgcn_make_buffer_rsrc((void*)(rp + lo), (short)0, nvec * 16, 0x00020000);
        const int voff = (int)threadIdx.x * 16;
        auto load = [&](int vi0) {
            return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rsrc, voff, vi0 * 16, 2));
        };
        // Initial bound from the exact maxima of the first batch.
        auto init_bound = [&](const u32x4 (&vec)[kUnroll]) {
            float mx = -INFINITY;
#pragma unroll
            for (int u = 0; u < kUnroll; ++u)
                mx = fmaxf(mx, u * kTopmThreads + (int)threadIdx.x < nvec ? Elem<T>::vmax(vec[u]) : -INFINITY);
            if (nvec >= kBatch) {
                // Every lane of the workgroup holds a full first batch: the 64th
                // largest of the 256 lane maxima is reached by 64 distinct
                // elements, so no key below it is in the top 64.
                const u64 k = wave_sort_desc((u64)f32_ord(mx) << 32);
                buf[lane] = k;
                __syncthreads();
                u64 l = k;
#pragma unroll
                for (int o = 1; o < kWaves; ++o)
                    l = wave_merge_top64(l, sbuf[(wave + o) % kWaves][kWave - 1 - lane]);
                __syncthreads();  // the key buffers are reused for admitted keys
                set_thr(w, bcast_u64(l, kWave - 1));
            } else if (__ballot((int)threadIdx.x < nvec) == ~0ull) {
                // 64 distinct elements (one per lane) reach the smallest lane maximum
                set_thr(w, (u64)f32_ord(-wave_max(-mx)) << 32);
                publish(w, &s_thr);
            }
        };
        // Evaluate the batch of vectors v0 + u * 256 + thread (u < kUnroll).
        auto process = [&](const u32x4 (&vec)[kUnroll], int v0) {
            float vm[kUnroll];
            set_thr(w, shared_bound(&s_thr));
            if (TAIL) tail_cover(ta, w.thr_val);
#pragma unroll
            for (int u = 0; u < kUnroll; ++u) vm[u] = Elem<T>::vfilter(vec[u]);
            if (v0 + kBatch > nvec) {  // last, partial batch
#pragma unroll
                for (int u = 0; u < kUnroll; ++u)
                    if (v0 + u * kTopmThreads + (int)threadIdx.x >= nvec) vm[u] = -INFINITY;
            }
#pragma unroll
            for (int u = 0; u < kUnroll; ++u) {
                const bool pass = vm[u] >= w.filt;
                if (TAIL && !pass && v0 + u * kTopmThreads + (int)threadIdx.x < nvec) {
                    // every element lies below the threshold: tail
#pragma unroll
                    for (int i = 0; i < P; ++i) tail_add_below(ta, Elem<T>::get(vec[u], i));
                }
                const u64 m = __ballot(pass);
                if (m == 0) continue;
                if (pass) {
                    const int pos = nst + prefix_count(m);
                    svec[wave][pos] = vec[u];
                    sidx[wave][pos] = v0 + u * kTopmThreads + (int)threadIdx.x;
                }
                nst += __popcll(m);
            }
            // fewer than 64 stay stashed between batches; none after the last
            const bool last = v0 + kBatch >= nvec;
            while (nst >= kWave || (last && nst > 0))
                drain_stash<T, TAIL>(w, ta, buf, &s_thr, svec[wave], sidx[wave], nst, lo);
        };
        // Software pipeline over two register sets: the next batch is in
        // flight while this one is evaluated, and no loaded register is
        // copied (a copy would wait for its load).
        u32x4 va[kUnroll], vb[kUnroll];
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) va[u] = load(u * kTopmThreads);
        for (int v0 = 0; v0 < nvec;) {
#pragma unroll
            for (int u = 0; u < kUnroll; ++u) vb[u] = load(v0 + kBatch + u * kTopmThreads);
            if (v0 == 0) init_bound(va);
            process(va, v0);
            v0 += kBatch;
            if (v0 >= nvec) break;
#pragma unroll
            for (int u = 0; u < kUnroll; ++u) va[u] = load(v0 + kBatch + u * kTopmThreads);
            process(vb, v0);
            v0 += kBatch;
        }
        tail_lo = lo + nvec * P;
    }
    // scalar part: the row's tail, or everything when rows are not 16-byte aligned
    for (int e0 = tail_lo; e0 < hi; e0 += kTopmThreads) {
        const int e = e0 + (int)threadIdx.x;
        const bool ok = e < hi;
        const float x = ok ? Elem<T>::scalar(rp + e) : -INFINITY;
        const bool cand = x >= w.thr_val;
        if (TAIL && ok && !cand) tail_add(ta, x);
        offer<TAIL>(w, ta, buf, &s_thr, ok && cand, topm_key(x, (uint32_t)e));
    }
    if (w.nbuf) fold_buffer<TAIL>(w, ta, buf, &s_thr);

    // merge the workgroup's four wave lists (reusing the key buffers)
    float tM = -FLT_MAX, tS = 0.f;
    if (TAIL) {
        tail_wave_total(ta, tM, tS);
        if (lane == 0) s_tail[wave] = float2{tM, tS};
    }
    __syncthreads();
    sbuf[wave][lane] = w.list;
    __syncthreads();
    if (wave == 0) {
        u64 l = w.list;
        TailAcc tb{-FLT_MAX, 0.f, tail_c};  // keys losing the merge, list entries past M
#pragma unroll
        for (int o = 1; o < kWaves; ++o) {
            const u64 other = sbuf[o][kWave - 1 - lane];
            if (TAIL) {
                const u64 lost = umin64(l, other);
                if (lost) tail_add(tb, topm_key_val(lost));
            }
            l = wave_merge_top64(l, other);
        }
        if (TAIL && nseg == 1 && lane >= M && l) tail_add(tb, topm_key_val(l));
        if (TAIL) {
#pragma unroll
            for (int o = 1; o < kWaves; ++o) tail_join(tM, tS, s_tail[o].x, s_tail[o].y);
            float m2, s2;
            tail_wave_total(tb, m2, s2);
            tail_join(tM, tS, m2, s2);
        }
        if (nseg == 1) {
            if (lane < M) {
                idx[(size_t)row * M + lane] = (int32_t)topm_key_id(l);
                val[(size_t)row * M + lane] = topm_key_val(l);
            }
            if (TAIL && lane == 0) tail_out[row] = tail_lse(tM, tS);
        } else {
            partial[((size_t)row * nseg + s) * kWave + lane] = l;
            if (TAIL && lane == 0) tail_part[(size_t)row * nseg + s] = float2{tM, tS};
        }
    }
}

// One wave per row: fold the row's `nseg` sorted partial lists, emit top M
// (and with TAIL the row's tail_lse: the segments' sums plus the keys losing
// this merge and the list entries past M).
template <bool TAIL>
__global__ __launch_bounds__(kWave) void topm_merge_kernel(const u64* __restrict__ partial, int nseg,
                                                           int M, int32_t* __restrict__ idx,
                                                           float* __restrict__ val, float tail_c,
                                                           const float2* __restrict__ tail_part,
                                                           float* __restrict__ tail_out) {
    const int row = blockIdx.x, lane = lane_id();
    const u64* p = partial + (size_t)row * nseg * kWave;
    u64 l = p[lane];
    TailAcc tb{-FLT_MAX, 0.f, tail_c};
    for (int s = 1; s < nseg; ++s) {
        const u64 other = p[(size_t)s * kWave + kWave - 1 - lane];
        if (TAIL) {
            const u64 lost = umin64(l, other);
            if (lost) tail_add(tb, topm_key_val(lost));
        }
        l = wave_merge_top64(l, other);
    }
    if (lane < M) {
        idx[(size_t)row * M + lane] = (int32_t)topm_key_id(l);
        val[(size_t)row * M + lane] = topm_key_val(l);
    }
    if (TAIL) {
        if (lane >= M && l) tail_add(tb, topm_key_val(l));
        float tM, tS;
        tail_wave_total(tb, tM, tS);
        for (int s = 0; s < nseg; ++s) {
            const float2 ps = tail_part[(size_t)row * nseg + s];
            tail_join(tM, tS, ps.x, ps.y);
        }
        if (lane == 0) tail_out[row] = tail_lse(tM, tS);
    }
}

}  // namespace

int topm_segments(int rows, int V) {
    // >= ~512 workgroups (2 per CU), segments of >= 16384 elements; fewer,
    // longer segments admit fewer keys (a running top-64 of N elements admits
    // about 64 ln(N / 64) of them per segment) and need no merge (measured on
    // 151936-wide bf16 rows: at 512 rows one segment per row beats two, at
    // 128 rows four beat eight)
    int want = (512 + rows - 1) / max(rows, 1);
    int cap = max(1, V / 16384);
    return max(1, min(want, cap));
}

hipError_t launch_topm(const void* base, int dtype, int rows, int V, int nseg, u64* partial,
                       int M, int32_t* idx, float* val, hipStream_t stream, LaunchEvents ev, float tail_c,
                       float* tail_out, float* tail_part, TopmSide side) {
    if (rows == 0) return hipSuccess;
    const size_t esz = dtype == 1 ? 2 : 4;
    const int per_vec = 16 / (int)esz;
    int seg = (V + nseg - 1) / nseg;
    seg = (seg + per_vec - 1) / per_vec * per_vec;  // segments start on vector boundaries
    const bool vec = ((uintptr_t)base % 16 == 0) && ((size_t)V * esz % 16 == 0);
    const dim3 grid(rows, nseg), block(kTopmThreads);
    float2* tp = reinterpret_cast<float2*>(tail_part);
    hipError_t e;
#define DT_TOPM(Ty, kV, TL) \
    launch_kernel(topm_partial_kernel<Ty, kV, TL>, grid, block, 0, stream, ev, (const Ty*)base, V, nseg, seg, \
                  partial, M, idx, val, tail_c, tail_out, tp, side)
    if (tail_out) {
        if (dtype == 1) e = vec ? DT_TOPM(bf16_t, true, true) : DT_TOPM(bf16_t, false, true);
        else e = vec ? DT_TOPM(float, true, true) : DT_TOPM(float, false, true);
    } else {
        if (dtype == 1) e = vec ? DT_TOPM(bf16_t, true, false) : DT_TOPM(bf16_t, false, false);
        else e = vec ? DT_TOPM(float, true, false) : DT_TOPM(float, false, false);
    }
#undef DT_TOPM
    if (e != hipSuccess) return e;
    if (nseg > 1) {
        if (tail_out)
            topm_merge_kernel<true><<<rows, kWave, 0, stream>>>(partial, nseg, M, idx, val, tail_c, tp, tail_out);
        else
            topm_merge_kernel<false><<<rows, kWave, 0, stream>>>(partial, nseg, M, idx, val, 0.f, nullptr, nullptr);
    }
    return hipGetLastError();
}

}  // namespace dt
