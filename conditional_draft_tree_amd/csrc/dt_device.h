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
// Cross-lane exchanges run on the VALU: DPP quad permutes and row shifts for
// lane distances 1..8, the gfx950 permlane swaps for 16 and 32 (no LDS
// traffic, no waits).  Lane semantics (checked on the device): row_shl:n
// reads lane i+n, row_shr:n reads lane i-n within a 16-lane row;
// permlane16_swap(v, v) = {row-even copies, row-odd copies} and
// permlane32_swap(v, v) = {lower-half copies, upper-half copies}; row_ror:n
// rotates a 16-lane row by n lanes.

__device__ __forceinline__ int lane_id() { return (int)(threadIdx.x & (kWave - 1)); }

template <int J>
__device__ __forceinline__ uint32_t xor_lane(uint32_t v) {
    const int lane = lane_id();
    if constexpr (J == 1) {
        return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0xB1, 0xF, 0xF, false);
    } else if constexpr (J == 2) {
        return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x4E, 0xF, 0xF, false);
    } else if constexpr (J == 4) {
        const uint32_t up = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x104, 0xF, 0xF, false);
        const uint32_t dn = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x114, 0xF, 0xF, false);
        return (lane & 4) ? dn : up;
    } else if constexpr (J == 8) {  // a rotation by 8 within the row: lane i ^ 8
        return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x128, 0xF, 0xF, false);
    } else if constexpr (J == 16) {
        const auto r = __builtin_amdgcn_permlane16_swap(v, v, false, false);
        return (lane & 16) ? r[0] : r[1];
    } else {
        static_assert(J == 32, "lane distance");
        const auto r = __builtin_amdgcn_permlane32_swap(v, v, false, false);
        return (lane & 32) ? r[0] : r[1];
    }
}
template <int J> __device__ __forceinline__ float xor_lane_f(float v) {
    return __uint_as_float(xor_lane<J>(__float_as_uint(v)));
}
template <int J> __device__ __forceinline__ u64 xor_lane_u64(u64 v) {
    return ((u64)xor_lane<J>((uint32_t)(v >> 32)) << 32) | (u64)xor_lane<J>((uint32_t)v);
}
__device__ __forceinline__ u64 xor_lane_u64(u64 v, int j) {
    switch (j) {
        case 1: return xor_lane_u64<1>(v);
        case 2: return xor_lane_u64<2>(v);
        case 4: return xor_lane_u64<4>(v);
        case 8: return xor_lane_u64<8>(v);
        case 16: return xor_lane_u64<16>(v);
        default: return xor_lane_u64<32>(v);
    }
}

// Value of lane `src` (wave-uniform index) in every lane.
// Lane i receives lane i-1's value; lane 0 receives 0 (DPP whole-wave shift
// right by one lane).
__device__ __forceinline__ u64 wave_shr1_u64(u64 v) {
    const uint32_t lo = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)(uint32_t)v, 0x138, 0xF, 0xF, false);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)(uint32_t)(v >> 32), 0x138, 0xF, 0xF, false);
    return ((u64)hi << 32) | lo;
}

__device__ __forceinline__ u64 bcast_u64(u64 v, int src) {
    const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(v >> 32), src);
    const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)v, src);
    return ((u64)hi << 32) | lo;
}

// All-reduce over the 64 lanes in the lane-distance order 32, 16, 8, 4, 2, 1
// (the xor butterfly).  At distances 32 and 16 both results of a swap hold
// the pair's two values, so a symmetric op takes them without a lane select;
// at distance 4 a rotation by 4 within the row stands in for the xor partner
// (after the distance-8 step lanes i and i ^ 8 hold the same value, and the
// rotation reads one of lanes i ^ 4, i ^ 12).  Every lane ends with the same
// bits, and with the bits of the plain butterfly: each step combines the same
// two values, in either order.
template <typename F>
__device__ __forceinline__ uint32_t wave_allreduce(uint32_t v, F op) {
    const auto a = __builtin_amdgcn_permlane32_swap(v, v, false, false);
    v = op(a[0], a[1]);
    const auto b = __builtin_amdgcn_permlane16_swap(v, v, false, false);
    v = op(b[0], b[1]);
    v = op(v, xor_lane<8>(v));
    v = op(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x124, 0xF, 0xF, false));  // row_ror:4
    v = op(v, xor_lane<2>(v));
    v = op(v, xor_lane<1>(v));
    return v;
}
__device__ __forceinline__ float wave_sum(float v) {
    return __uint_as_float(wave_allreduce(__float_as_uint(v), [](uint32_t x, uint32_t y) {
        return __float_as_uint(__uint_as_float(x) + __uint_as_float(y));
    }));
}
__device__ __forceinline__ float wave_max(float v) {
    return __uint_as_float(wave_allreduce(__float_as_uint(v), [](uint32_t x, uint32_t y) {
        return __float_as_uint(fmaxf(__uint_as_float(x), __uint_as_float(y)));
    }));
}
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
    return wave_allreduce(v, [](uint32_t x, uint32_t y) { return x > y ? x : y; });
}
__device__ __forceinline__ u64 umax64(u64 a, u64 b) { return a > b ? a : b; }
__device__ __forceinline__ u64 umin64(u64 a, u64 b) { return a > b ? b : a; }
// Largest 64-bit key over the 64 lanes: the largest high word, and when more
// than one lane holds it, the largest low word among those lanes.
__device__ __forceinline__ u64 wave_max_u64(u64 v) {
    const uint32_t hi = (uint32_t)(v >> 32);
    const uint32_t mh = wave_max_u32(hi);
    const u64 tied = __ballot(hi == mh);
    if (__builtin_popcountll(tied) == 1) return bcast_u64(v, (int)__builtin_ctzll(tied));  // (uniform)
    return ((u64)mh << 32) | wave_max_u32(hi == mh ? (uint32_t)v : 0u);
}

// One compare-exchange stage of a bitonic network at lane distance J:
// the lower lane of each pair keeps the larger key when `desc`.
template <int J>
__device__ __forceinline__ u64 bitonic_stage(u64 key, bool desc) {
    const u64 o = xor_lane_u64<J>(key);
    const bool lower = (lane_id() & J) == 0;
    return (lower == desc) ? umax64(key, o) : umin64(key, o);
}

// Bitonic sort of one key per lane into descending lane order (ascending
// when `ascending`).
__device__ __forceinline__ u64 wave_sort(u64 key, bool ascending) {
    const int lane = lane_id();
#define DT_STAGE(K, J) key = bitonic_stage<J>(key, (((lane & K) == 0) != ascending))
    DT_STAGE(2, 1);
    DT_STAGE(4, 2); DT_STAGE(4, 1);
    DT_STAGE(8, 4); DT_STAGE(8, 2); DT_STAGE(8, 1);
    DT_STAGE(16, 8); DT_STAGE(16, 4); DT_STAGE(16, 2); DT_STAGE(16, 1);
    DT_STAGE(32, 16); DT_STAGE(32, 8); DT_STAGE(32, 4); DT_STAGE(32, 2); DT_STAGE(32, 1);
    DT_STAGE(64, 32); DT_STAGE(64, 16); DT_STAGE(64, 8); DT_STAGE(64, 4); DT_STAGE(64, 2); DT_STAGE(64, 1);
#undef DT_STAGE
    return key;
}
__device__ __forceinline__ u64 wave_sort_desc(u64 key) { return wave_sort(key, false); }

// Finish a bitonic sequence into descending lane order.
__device__ __forceinline__ u64 wave_bitonic_merge_desc(u64 key) {
    key = bitonic_stage<32>(key, true);
    key = bitonic_stage<16>(key, true);
    key = bitonic_stage<8>(key, true);
    key = bitonic_stage<4>(key, true);
    key = bitonic_stage<2>(key, true);
    key = bitonic_stage<1>(key, true);
    return key;
}

// `list` sorted descending and `other_asc` sorted ascending across the wave:
// the 64 largest keys of both, sorted descending.
__device__ __forceinline__ u64 wave_merge_top64(u64 list, u64 other_asc) {
    return wave_bitonic_merge_desc(umax64(list, other_asc));  // bitonic, holds the top 64
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
                                          const void* b_hh, int dtype, int H, int k, float hprev);

// Four consecutive parameter elements [i, i+4) (zeros when p is NULL).
typedef float dt_f32x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ dt_f32x4 load_param4(const void* p, int dtype, size_t i) {
    if (!p) return dt_f32x4{0.f, 0.f, 0.f, 0.f};
    if (dtype == 1) {
        const uint2 w = *reinterpret_cast<const uint2*>((const uint16_t*)p + i);
        return dt_f32x4{__uint_as_float(w.x << 16), __uint_as_float(w.x & 0xFFFF0000u),
                        __uint_as_float(w.y << 16), __uint_as_float(w.y & 0xFFFF0000u)};
    }
    return *reinterpret_cast<const dt_f32x4*>((const float*)p + i);
}

// GRU cell with the biases already loaded (bi*: input biases, bh*: hidden).
__device__ __forceinline__ float gru_cell_b(float sr, float sz, float snx, float snh, float bir,
                                            float biz, float bin, float bhr, float bhz, float bhn,
                                            float hprev) {
    const float r = 1.f / (1.f + expf(-(sr + (bir + bhr))));
    const float u = 1.f / (1.f + expf(-(sz + (biz + bhz))));
    const float c = tanhf((snx + bin) + r * (snh + bhn));
    return (1.f - u) * c + u * hprev;
}

// GRU elementwise update of hidden unit k from its gate sums (biases not
// yet added): reset r, update u, candidate c; h' = (1 - u) c + u h.
__device__ __forceinline__ float gru_cell(float sr, float sz, float snx, float snh, const void* b_ih,
                                          const void* b_hh, int dtype, int H, int k, float hprev) {
    return gru_cell_b(sr, sz, snx, snh, load_param(b_ih, dtype, k), load_param(b_ih, dtype, H + k),
                      load_param(b_ih, dtype, 2 * H + k), load_param(b_hh, dtype, k),
                      load_param(b_hh, dtype, H + k), load_param(b_hh, dtype, 2 * H + k), hprev);
}

// Partial-sum buffer of the gate contraction: [ksplit][B][kGateSlots][H],
// slots 0 reset, 1 update, 2 candidate (x part), 3 candidate (h part).
constexpr int kGateSlots = 4;
constexpr int kMaxKsplit = 6;  // K ranges of the gate contraction

// New state of (row b, unit k): the K-range partials added in K order.
__device__ __forceinline__ float gru_from_partials(const float* partial, int ksplit, int B, int b,
                                                   int H, int k, const void* b_ih, const void* b_hh,
                                                   int dtype, float hprev) {
    float t[4] = {0.f, 0.f, 0.f, 0.f};
    for (int s = 0; s < ksplit; ++s) {
        const float* p = partial + ((size_t)(s * B + b) * kGateSlots) * H + k;
#pragma unroll
        for (int g = 0; g < 4; ++g) t[g] += p[(size_t)g * H];
    }
    return gru_cell(t[0], t[1], t[2], t[3], b_ih, b_hh, dtype, H, k, hprev);
}

// x = p[0] + p[1] + p[2] exactly, each part a bf16 (bits returned): the
// first two parts are x and the first remainder cut to their leading 8
// significant bits (the high half of the word), every subtraction is exact,
// and the last remainder has at most 8 significant bits (as long as it is not
// below bf16's subnormal range: |x| >= 2^-110 or x = 0).
__device__ __forceinline__ void split3_bf16(float x, uint32_t p[3]) {
    const uint32_t b0 = __float_as_uint(x) & 0xFFFF0000u;
    const float r1 = x - __uint_as_float(b0);
    const uint32_t b1 = __float_as_uint(r1) & 0xFFFF0000u;
    const float r2 = r1 - __uint_as_float(b1);
    p[0] = b0 >> 16;
    p[1] = b1 >> 16;
    p[2] = __float_as_uint(r2) >> 16;
}

}  // namespace dt
