// topm.hip -- top-M marginal candidates per (request, block position) row.
//
// The builder precomputes the top-M marginal tokens of every depth before the
// expansion ([captcha] "Methodology -- deep read"; [gist] "Composants clés --
// Restriction de candidats (Top-M)").  Order: value desc, token id asc.
//
// The select is HBM-bound: every row of V logits is streamed once, in
// `nseg` segments of one 256-thread workgroup each.  Every wave keeps the 64
// best (value, ~id) keys it has admitted, sorted across its lanes, and an
// admission threshold: a key below it cannot be among the segment's 64 best.
// Valid thresholds come from (a) the minimum of the 64 lane maxima of the
// first vectors (64 distinct elements reach it), (b) the wave's own 64th best
// key, and (c) the best value threshold any wave of the workgroup has
// published in LDS (the segment's list merges all four waves).  The hot loop
// is one max-reduction and one compare per 16-byte vector; a vector whose
// maximum reaches the threshold is stashed in LDS, and stashed vectors are
// evaluated 64 at a time (one per lane), which amortizes the wave-wide work of
// admitting a key.  Admitted keys are folded into the list with a bitonic
// sort + merge.  topm_merge folds a row's partial lists into its top M.
#include "dt_device.h"
#include "dt_launch.h"

namespace dt {

namespace {

constexpr int kTopmThreads = 256;
constexpr int kWaves = kTopmThreads / kWave;
constexpr int kUnroll = 8;   // 16-byte vectors in flight per lane
constexpr int kStash = 128;  // stashed vectors per wave

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
    __device__ static float scalar(const bf16_t* p) { return bf16_to_f32(*p); }
};

// Per-wave running top-64: `list` (one key per lane, descending), a staging
// buffer of admitted keys in LDS and the admission threshold `thr` (keys
// below it are rejected; 0 admits everything).
struct WaveTop {
    u64 list;
    u64 thr;
    float thr_val;  // value part of thr (-inf while thr == 0)
    int nbuf;
};

__device__ __forceinline__ void set_thr(WaveTop& w, u64 t) {
    if (t > w.thr) {
        w.thr = t;
        w.thr_val = topm_key_val(t);
    }
}

// Publish the value part of the wave's threshold to the workgroup.
__device__ __forceinline__ void publish(const WaveTop& w, uint32_t* s_thr) {
    if (w.thr && lane_id() == 0) atomicMax(s_thr, (uint32_t)(w.thr >> 32));
}

__device__ __forceinline__ void fold_buffer(WaveTop& w, u64* buf, uint32_t* s_thr) {
    const int lane = lane_id();
    u64 x = lane < w.nbuf ? buf[lane] : 0ull;
    x = wave_sort(x, /*ascending=*/true);
    w.list = wave_merge_top64(w.list, x);
    w.nbuf = 0;
    set_thr(w, bcast_u64(w.list, kWave - 1));
    publish(w, s_thr);
}

// Offer one key per lane (valid only where `ok`); wave-uniform call.
__device__ __forceinline__ void offer(WaveTop& w, u64* buf, uint32_t* s_thr, bool ok, u64 key) {
    bool pass = ok && key >= w.thr;
    u64 m = __ballot(pass);
    if (m == 0) return;
    int cnt = __popcll(m);
    if (w.nbuf + cnt > kWave) {
        fold_buffer(w, buf, s_thr);
        pass = ok && key >= w.thr;
        m = __ballot(pass);
        cnt = __popcll(m);
    }
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

// Evaluate the first min(nst, 64) stashed vectors (one per lane) element by
// element, then move the rest down.
template <typename T>
__device__ __forceinline__ void drain_stash(WaveTop& w, u64* buf, uint32_t* s_thr, u32x4* svec,
                                            int* sidx, int& nst, int lo) {
    constexpr int P = Elem<T>::kPerVec;
    const int lane = lane_id();
    const int take = min(nst, kWave);
    const bool on = lane < take;
    const u32x4 v = on ? svec[lane] : u32x4{0u, 0u, 0u, 0u};
    const int vi = on ? sidx[lane] : 0;
    set_thr(w, (u64)__hip_atomic_load(s_thr, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP) << 32);
#pragma unroll
    for (int i = 0; i < P; ++i) {
        const float x = Elem<T>::get(v, i);
        offer(w, buf, s_thr, on && x >= w.thr_val, topm_key(x, (uint32_t)(lo + vi * P + i)));
    }
    const int rest = nst - take;
    u32x4 mv = u32x4{0u, 0u, 0u, 0u};
    int mi = 0;
    if (lane < rest) {
        mv = svec[kWave + lane];
        mi = sidx[kWave + lane];
    }
    __builtin_amdgcn_wave_barrier();
    if (lane < rest) {
        svec[lane] = mv;
        sidx[lane] = mi;
    }
    nst = rest;
}

template <typename T, bool kVec>
__global__ __launch_bounds__(kTopmThreads) void topm_partial_kernel(const T* __restrict__ base, int V,
                                                                    int nseg, int seg,
                                                                    u64* __restrict__ partial) {
    __shared__ u64 sbuf[kWaves][kWave];
    __shared__ u32x4 svec[kWaves][kStash];
    __shared__ int sidx[kWaves][kStash];
    __shared__ uint32_t s_thr;
    const int row = blockIdx.y, s = blockIdx.x;
    const int wave = threadIdx.x / kWave, lane = lane_id();
    const T* rp = base + (size_t)row * (size_t)V;
    const int lo = s * seg;
    const int hi = min(V, lo + seg);
    u64* buf = sbuf[wave];
    if (threadIdx.x == 0) s_thr = 0u;
    __syncthreads();

    WaveTop w;
    w.list = 0ull;
    w.thr = 0ull;
    w.thr_val = -INFINITY;
    w.nbuf = 0;
    int nst = 0;

    int tail_lo = lo;
    if (kVec && hi > lo) {
        constexpr int P = Elem<T>::kPerVec;
        const int nvec = (hi - lo) / P;
        const u32x4* vp = reinterpret_cast<const u32x4*>(rp + lo);
        bool first = true;
        for (int v0 = 0; v0 < nvec; v0 += kUnroll * kTopmThreads) {
            u32x4 vec[kUnroll];
            float vm[kUnroll];
            bool ok[kUnroll];
#pragma unroll
            for (int u = 0; u < kUnroll; ++u) {
                const int vi = v0 + u * kTopmThreads + (int)threadIdx.x;
                ok[u] = vi < nvec;
                vec[u] = ok[u] ? __builtin_nontemporal_load(vp + vi) : u32x4{0u, 0u, 0u, 0u};
            }
#pragma unroll
            for (int u = 0; u < kUnroll; ++u) vm[u] = ok[u] ? Elem<T>::vmax(vec[u]) : -INFINITY;
            if (first) {
                // 64 distinct elements (one per lane) reach the smallest lane maximum
                first = false;
                float mx = vm[0];
#pragma unroll
                for (int u = 1; u < kUnroll; ++u) mx = fmaxf(mx, vm[u]);
                if (__ballot(v0 + (int)threadIdx.x < nvec) == ~0ull) {
                    set_thr(w, (u64)f32_ord(-wave_max(-mx)) << 32);
                    publish(w, &s_thr);
                }
            } else {
                set_thr(w, (u64)__hip_atomic_load(&s_thr, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP) << 32);
            }
#pragma unroll
            for (int u = 0; u < kUnroll; ++u) {
                const bool pass = ok[u] && vm[u] >= w.thr_val;
                const u64 m = __ballot(pass);
                if (m == 0) continue;
                if (pass) {
                    const int pos = nst + prefix_count(m);
                    svec[wave][pos] = vec[u];
                    sidx[wave][pos] = v0 + u * kTopmThreads + (int)threadIdx.x;
                }
                nst += __popcll(m);
                if (nst >= kWave) drain_stash<T>(w, buf, &s_thr, svec[wave], sidx[wave], nst, lo);
            }
        }
        while (nst > 0) drain_stash<T>(w, buf, &s_thr, svec[wave], sidx[wave], nst, lo);
        tail_lo = lo + nvec * P;
    }
    // scalar part: the row's tail, or everything when rows are not 16-byte aligned
    for (int e0 = tail_lo; e0 < hi; e0 += kTopmThreads) {
        const int e = e0 + (int)threadIdx.x;
        const bool ok = e < hi;
        const float x = ok ? Elem<T>::scalar(rp + e) : -INFINITY;
        offer(w, buf, &s_thr, ok && x >= w.thr_val, topm_key(x, (uint32_t)e));
    }
    if (w.nbuf) fold_buffer(w, buf, &s_thr);

    // merge the workgroup's four wave lists (reusing the key buffers)
    __syncthreads();
    sbuf[wave][lane] = w.list;
    __syncthreads();
    if (wave == 0) {
        u64 l = w.list;
#pragma unroll
        for (int o = 1; o < kWaves; ++o) l = wave_merge_top64(l, sbuf[o][kWave - 1 - lane]);
        partial[((size_t)row * nseg + s) * kWave + lane] = l;
    }
}

// One wave per row: fold the row's `nseg` sorted partial lists, emit top M.
__global__ __launch_bounds__(kWave) void topm_merge_kernel(const u64* __restrict__ partial, int nseg,
                                                           int M, int32_t* __restrict__ idx,
                                                           float* __restrict__ val) {
    const int row = blockIdx.x, lane = lane_id();
    const u64* p = partial + (size_t)row * nseg * kWave;
    u64 l = p[lane];
    for (int s = 1; s < nseg; ++s) l = wave_merge_top64(l, p[(size_t)s * kWave + kWave - 1 - lane]);
    if (lane < M) {
        idx[(size_t)row * M + lane] = (int32_t)topm_key_id(l);
        val[(size_t)row * M + lane] = topm_key_val(l);
    }
}

}  // namespace

int topm_segments(int rows, int V) {
    // >= ~1024 workgroups (4 per CU), segments of >= 16384 elements; fewer,
    // longer segments admit fewer keys (a running top-64 of N elements admits
    // about 64 ln(N / 64) of them per segment)
    int want = (1024 + rows - 1) / max(rows, 1);
    int cap = max(1, V / 16384);
    return max(1, min(want, cap));
}

hipError_t launch_topm(const void* base, int dtype, int rows, int V, int nseg, u64* partial,
                       int M, int32_t* idx, float* val, hipStream_t stream, hipEvent_t ev_mid) {
    if (rows == 0) return hipSuccess;
    const size_t esz = dtype == 1 ? 2 : 4;
    const int per_vec = 16 / (int)esz;
    int seg = (V + nseg - 1) / nseg;
    seg = (seg + per_vec - 1) / per_vec * per_vec;  // segments start on vector boundaries
    const bool vec = ((uintptr_t)base % 16 == 0) && ((size_t)V * esz % 16 == 0);
    dim3 grid(nseg, rows);
    if (dtype == 1) {
        if (vec)
            topm_partial_kernel<bf16_t, true><<<grid, kTopmThreads, 0, stream>>>((const bf16_t*)base, V, nseg, seg, partial);
        else
            topm_partial_kernel<bf16_t, false><<<grid, kTopmThreads, 0, stream>>>((const bf16_t*)base, V, nseg, seg, partial);
    } else {
        if (vec)
            topm_partial_kernel<float, true><<<grid, kTopmThreads, 0, stream>>>((const float*)base, V, nseg, seg, partial);
        else
            topm_partial_kernel<float, false><<<grid, kTopmThreads, 0, stream>>>((const float*)base, V, nseg, seg, partial);
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    if (ev_mid) {
        e = hipEventRecord(ev_mid, stream);
        if (e != hipSuccess) return e;
    }
    topm_merge_kernel<<<rows, kWave, 0, stream>>>(partial, nseg, M, idx, val);
    return hipGetLastError();
}

}  // namespace dt
