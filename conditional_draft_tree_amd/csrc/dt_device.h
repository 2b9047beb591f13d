// dt_device.h -- device helpers and launch plan shared by the library's HIP
// sources (gfx950, wave64).  Internal; not part of the C ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace dt {

typedef unsigned long long u64;
typedef uint16_t bf16_t;  // bfloat16 bit pattern

constexpr int kWave = 64;
constexpr int kMaxM = 64;  // one candidate per lane
constexpr int kMaxN = 64;  // queue fits one wave (see the node kernel)
constexpr int kMaxH = 4096;

// ---------------------------------------------------------------- scalars --

__device__ __forceinline__ float bf16_to_f32(uint32_t bits16) {
    return __uint_as_float(bits16 << 16);
}

// binary32 -> bf16 bits, round to nearest, ties to even (finite inputs).
__device__ __forceinline__ uint32_t f32_to_bf16_rne(float f) {
    uint32_t u = __float_as_uint(f);
    u += 0x7FFFu + ((u >> 16) & 1u);
    return u >> 16;
}

// Monotone map of binary32 bit patterns to unsigned integers (a < b as floats
// <=> ord(a) < ord(b) as integers), with -0 folded onto +0.
__device__ __forceinline__ uint32_t f32_ord(float f) {
    uint32_t u = __float_as_uint(f);
    if (u == 0x80000000u) u = 0u;
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float f32_unord(uint32_t o) {
    uint32_t u = (o & 0x80000000u) ? (o & 0x7FFFFFFFu) : ~o;
    return __uint_as_float(u);
}

// Candidate key of the top-M select: value first, then the LOWER token id.
__device__ __forceinline__ u64 topm_key(float v, uint32_t id) {
    return ((u64)f32_ord(v) << 32) | (u64)(0xFFFFFFFFu - id);
}
__device__ __forceinline__ uint32_t topm_key_id(u64 k) { return 0xFFFFFFFFu - (uint32_t)k; }
__device__ __forceinline__ float topm_key_val(u64 k) { return f32_unord((uint32_t)(k >> 32)); }

// Queue key of a candidate node: score desc, depth asc, parent slot asc,
// sibling rank asc -- a larger key is popped first.  depth 1..64,
// parent 0..63, rank 0..63.  Key 0 marks an empty queue slot.
__device__ __forceinline__ u64 queue_key(float score, int depth, int parent, int rank) {
    uint32_t lo = ((uint32_t)(127 - depth) << 13) | ((uint32_t)(127 - parent) << 6) |
                  (uint32_t)(63 - rank);
    return ((u64)f32_ord(score) << 32) | lo;
}
__device__ __forceinline__ float qk_score(u64 k) { return f32_unord((uint32_t)(k >> 32)); }
__device__ __forceinline__ int qk_depth(u64 k) { return 127 - (int)(((uint32_t)k >> 13) & 127u); }
__device__ __forceinline__ int qk_parent(u64 k) { return 127 - (int)(((uint32_t)k >> 6) & 127u); }
__device__ __forceinline__ int qk_rank(u64 k) { return 63 - (int)((uint32_t)k & 63u); }

// Child key of the per-node sort: log-prob desc, then the LOWER token id.
__device__ __forceinline__ u64 child_key(float lp, int tok) {
    return ((u64)f32_ord(lp) << 32) | (u64)(0xFFFFFFFFu - (uint32_t)tok);
}

// ------------------------------------------------------------ wave ops ----

__device__ __forceinline__ int lane_id() { return (int)(threadIdx.x & (kWave - 1)); }

__device__ __forceinline__ u64 shfl_xor_u64(u64 v, int m) {
    return (u64)__shfl_xor((unsigned long long)v, m, kWave);
}
__device__ __forceinline__ u64 shfl_u64(u64 v, int src) {
    return (u64)__shfl((unsigned long long)v, src, kWave);
}

// Sum over the 64 lanes; the butterfly order is fixed, so the result is
// reproducible and identical in every lane.
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m, kWave);
    return v;
}
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) v = fmaxf(v, __shfl_xor(v, m, kWave));
    return v;
}
__device__ __forceinline__ u64 wave_max_u64(u64 v) {
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) {
        u64 o = shfl_xor_u64(v, m);
        v = o > v ? o : v;
    }
    return v;
}

// Bitonic sort of one key per lane into descending lane order.
__device__ __forceinline__ u64 wave_sort_desc(u64 key) {
    const int lane = lane_id();
#pragma unroll
    for (int k = 2; k <= kWave; k <<= 1) {
#pragma unroll
        for (int j = k >> 1; j > 0; j >>= 1) {
            u64 o = shfl_xor_u64(key, j);
            bool desc = (lane & k) == 0;
            bool lower = (lane & j) == 0;
            u64 mx = o > key ? o : key, mn = o > key ? key : o;
            key = (lower == desc) ? mx : mn;
        }
    }
    return key;
}

// Finish a bitonic sequence into descending lane order.
__device__ __forceinline__ u64 wave_bitonic_merge_desc(u64 key) {
    const int lane = lane_id();
#pragma unroll
    for (int j = kWave >> 1; j > 0; j >>= 1) {
        u64 o = shfl_xor_u64(key, j);
        bool lower = (lane & j) == 0;
        u64 mx = o > key ? o : key, mn = o > key ? key : o;
        key = lower ? mx : mn;
    }
    return key;
}

// `list` and `other` are each sorted descending across the wave; returns the
// 64 largest keys of both, sorted descending.
__device__ __forceinline__ u64 wave_merge_top64(u64 list, u64 other_sorted) {
    u64 rev = shfl_u64(other_sorted, kWave - 1 - lane_id());
    u64 m = rev > list ? rev : list;  // bitonic, holds the top 64
    return wave_bitonic_merge_desc(m);
}

}  // namespace dt

namespace dt {

// A parameter vector element (binary32 or bf16 storage), 0 when p is NULL.
__device__ __forceinline__ float load_param(const void* p, int dtype, size_t i) {
    if (!p) return 0.f;
    return dtype == 1 ? bf16_to_f32(((const uint16_t*)p)[i]) : ((const float*)p)[i];
}

// GRU elementwise update of hidden unit k from its gate sums (bias not yet
// added): reset r, update u, candidate c; h' = (1 - u) c + u h.
__device__ __forceinline__ float gru_cell(float sr, float sz, float snx, float snh, const void* b_ih,
                                          const void* b_hh, int dtype, int H, int k, float hprev) {
    sr += load_param(b_ih, dtype, k) + load_param(b_hh, dtype, k);
    sz += load_param(b_ih, dtype, H + k) + load_param(b_hh, dtype, H + k);
    snx += load_param(b_ih, dtype, 2 * H + k);
    snh += load_param(b_hh, dtype, 2 * H + k);
    const float r = 1.f / (1.f + expf(-sr));
    const float u = 1.f / (1.f + expf(-sz));
    const float c = tanhf(snx + r * snh);
    return (1.f - u) * c + u * hprev;
}

// Partial-sum buffer of the gate contraction: [ksplit][B][kGateSlots][H],
// slots 0 reset, 1 update, 2 candidate (x part), 3 candidate (h part), 4 the
// previous state (K range 0 only).
constexpr int kGateSlots = 5;

// New state of (row b, unit k): the K-range partials added in K order.
__device__ __forceinline__ float gru_from_partials(const float* partial, int ksplit, int B, int b,
                                                   int H, int k, const void* b_ih, const void* b_hh,
                                                   int dtype) {
    float t[4] = {0.f, 0.f, 0.f, 0.f};
    for (int s = 0; s < ksplit; ++s) {
        const float* p = partial + ((size_t)(s * B + b) * kGateSlots) * H + k;
#pragma unroll
        for (int g = 0; g < 4; ++g) t[g] += p[(size_t)g * H];
    }
    const float hprev = partial[((size_t)b * kGateSlots + 4) * H + k];
    return gru_cell(t[0], t[1], t[2], t[3], b_ih, b_hh, dtype, H, k, hprev);
}

// x = p[0] + p[1] + p[2] exactly, each part a bf16 (bits returned): every
// subtraction below is exact, and the last remainder has at most 8
// significant bits.
__device__ __forceinline__ void split3_bf16(float x, uint32_t p[3]) {
    float r = x;
#pragma unroll
    for (int s = 0; s < 3; ++s) {
        p[s] = f32_to_bf16_rne(r);
        r = r - bf16_to_f32(p[s]);
    }
}

}  // namespace dt
