// topm.hip -- top-M marginal candidates per (request, block position) row.
//
// The builder precomputes the top-M marginal tokens of every depth before the
// expansion ([captcha] "Methodology -- deep read"; [gist] "Composants clés --
// Restriction de candidats (Top-M)").  Order: value desc, token id asc.
//
// The select is HBM-bound: every row of V logits is streamed once.  Each
// row is split into `nseg` segments, one 256-thread workgroup per segment;
// every lane streams 16-byte vectors, and its wave keeps the 64 best
// (value, ~id) keys seen so far sorted across its 64 lanes.  A vector is
// inspected element by element only when its maximum reaches the wave's
// current 64th-best value; for a row drawn in random order that happens for
// O(64 ln(V/64)) elements, so the common path is one max-reduction and one
// compare per vector.  Candidates go to a 64-entry LDS buffer per wave and
// are folded into the list with a bitonic sort + merge when it fills.  The
// four wave lists of a workgroup are merged into one partial list per
// segment; topm_merge folds a row's partial lists into its top M.
#include "dt_device.h"
#include "dt_launch.h"

namespace dt {

namespace {

constexpr int kTopmThreads = 256;
constexpr int kUnroll = 4;  // 16-byte vectors in flight per lane

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

template <typename T> struct Elem;
template <> struct Elem<float> {
    static constexpr int kPerVec = 4;
    __device__ static float get(const u32x4& v, int i) {
        const uint32_t w[4] = {v.x, v.y, v.z, v.w};
        return __uint_as_float(w[i]);
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
        const uint32_t w[4] = {v.x, v.y, v.z, v.w};
        uint32_t x = w[i >> 1];
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
// buffer in LDS and the current admission threshold (the 64th best key; 0
// while the list is not full).
struct WaveTop {
    u64 list;
    u64 thr;
    float thr_val;  // value part of thr; -inf while the list is not full
    int nbuf;
};

__device__ __forceinline__ void fold_buffer(WaveTop& w, u64* buf) {
    const int lane = lane_id();
    u64 x = lane < w.nbuf ? buf[lane] : 0ull;
    x = wave_sort_desc(x);
    w.list = wave_merge_top64(w.list, x);
    w.nbuf = 0;
    w.thr = shfl_u64(w.list, kWave - 1);
    w.thr_val = w.thr ? topm_key_val(w.thr) : -INFINITY;
}

// Offer one key per lane (valid only where `ok`); wave-uniform call.
__device__ __forceinline__ void offer(WaveTop& w, u64* buf, bool ok, u64 key) {
    bool pass = ok && key > w.thr;
    u64 m = __ballot(pass);
    if (m == 0) return;
    int cnt = __popcll(m);
    if (w.nbuf + cnt > kWave) {
        fold_buffer(w, buf);
        pass = ok && key > w.thr;
        m = __ballot(pass);
        cnt = __popcll(m);
    }
    if (pass) {
        int pos = w.nbuf + (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32),
                                                          __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
        buf[pos] = key;
    }
    w.nbuf += cnt;
}

template <typename T, bool kVec>
__global__ __launch_bounds__(kTopmThreads) void topm_partial_kernel(const T* __restrict__ base, int V,
                                                                    int nseg, int seg,
                                                                    u64* __restrict__ partial) {
    __shared__ u64 sbuf[kTopmThreads / kWave][kWave];
    __shared__ u64 slist[kTopmThreads / kWave][kWave];
    const int row = blockIdx.y, s = blockIdx.x;
    const int wave = threadIdx.x / kWave, lane = lane_id();
    const T* rp = base + (size_t)row * (size_t)V;
    const int lo = s * seg;
    const int hi = min(V, lo + seg);
    u64* buf = sbuf[wave];

    WaveTop w;
    w.list = 0ull;
    w.thr = 0ull;
    w.thr_val = -INFINITY;
    w.nbuf = 0;

    int tail_lo = lo;
    if (kVec && hi > lo) {
        constexpr int P = Elem<T>::kPerVec;
        const int nvec = (hi - lo) / P;
        const u32x4* vp = reinterpret_cast<const u32x4*>(rp + lo);
        // each block-iteration covers kUnroll * 256 consecutive vectors
        for (int v0 = 0; v0 < nvec; v0 += kUnroll * kTopmThreads) {
            u32x4 vec[kUnroll];
            bool ok[kUnroll];
#pragma unroll
            for (int u = 0; u < kUnroll; ++u) {
                int vi = v0 + u * kTopmThreads + (int)threadIdx.x;
                ok[u] = vi < nvec;
                vec[u] = ok[u] ? __builtin_nontemporal_load(vp + vi) : u32x4{0u, 0u, 0u, 0u};
            }
            float mx = -INFINITY;
#pragma unroll
            for (int u = 0; u < kUnroll; ++u)
                if (ok[u]) mx = fmaxf(mx, Elem<T>::vmax(vec[u]));
            if (__ballot(mx >= w.thr_val) == 0) continue;
            // slow path: exact keys of every element that may enter
#pragma unroll
            for (int u = 0; u < kUnroll; ++u) {
                int vi = v0 + u * kTopmThreads + (int)threadIdx.x;
#pragma unroll
                for (int i = 0; i < P; ++i) {
                    float x = Elem<T>::get(vec[u], i);
                    bool cand = ok[u] && x >= w.thr_val;
                    uint32_t id = (uint32_t)(lo + vi * P + i);
                    offer(w, buf, cand, topm_key(x, id));
                }
            }
        }
        tail_lo = lo + nvec * P;
    }
    // scalar part: the row's tail, or everything when rows are not 16-byte aligned
    for (int e0 = tail_lo; e0 < hi; e0 += kTopmThreads) {
        int e = e0 + (int)threadIdx.x;
        bool ok = e < hi;
        float x = ok ? Elem<T>::scalar(rp + e) : -INFINITY;
        offer(w, buf, ok && x >= w.thr_val, topm_key(x, (uint32_t)e));
    }
    if (w.nbuf) fold_buffer(w, buf);

    // merge the workgroup's four wave lists
    slist[wave][lane] = w.list;
    __syncthreads();
    if (wave == 0) {
        u64 l = w.list;
#pragma unroll
        for (int o = 1; o < kTopmThreads / kWave; ++o) l = wave_merge_top64(l, slist[o][lane]);
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
    for (int s = 1; s < nseg; ++s) l = wave_merge_top64(l, p[(size_t)s * kWave + lane]);
    if (lane < M) {
        idx[(size_t)row * M + lane] = (int32_t)topm_key_id(l);
        val[(size_t)row * M + lane] = topm_key_val(l);
    }
}

}  // namespace

int topm_segments(int rows, int V) {
    // aim for >= ~4096 workgroups (16 per CU), segments of >= 8192 elements
    int want = (4096 + rows - 1) / max(rows, 1);
    int cap = max(1, V / 8192);
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
