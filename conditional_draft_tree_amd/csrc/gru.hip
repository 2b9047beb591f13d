// gru.hip -- the GRU gate contraction of one expansion step, batched over the
// B requests.
//
// Expanding a node advances the GRU hidden state along the node's path with
// its realized token ([captcha] "Methodology -- deep read"; [gist] "Composants
// clés": only the light GRU correction is recomputed per node).  Every request
// pops exactly one node per step, so the B updates of a step form one
// contraction [B, E+H] x [E+H, 3H].  The reset and update gates sum the x and
// h parts; the candidate gate keeps them apart (its h part is scaled by the
// reset gate), hence four gate sums per output.
//
// bf16 path (v_mfma_f32_16x16x32_bf16, binary32 accumulation).  A workgroup
// owns 16 hidden units x 64 rows x one of `ksplit` K ranges; its four waves
// take a quarter of that range each, over all 64 rows, so every weight element
// is loaded by exactly one wave.  The waves' sums meet in LDS in wave order and
// the workgroup writes its K-range partial sums; the consumer (the node step,
// or gru_finalize) adds the `ksplit` partials in K order and applies the GRU
// cell.  The binary32 state h is fed as the exact sum of three bf16 parts
// (computed once per state by its producer), so the recurrent product is not
// quantized.  The K-range-0 workgroups also copy the previous state into the
// partial buffer, so the consumer needs no dependent load.
#include "dt_device.h"
#include "dt_launch.h"

namespace dt {

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;
constexpr int kRowBlocks = 4;  // 4 x 16 rows per workgroup

__device__ __forceinline__ bf16x8 load_bf16x8(const bf16_t* p) {
    return __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(p));
}

__device__ __forceinline__ f32x4 mfma(bf16x8 a, bf16x8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__global__ __launch_bounds__(kThreads) void gru_gates_bf16_kernel(GruGatesArgs a) {
    __shared__ float red[kThreads / kWave - 1][kRowBlocks * 4 * 4][kWave];  // 48 KB
    const int wave = threadIdx.x / kWave, lane = lane_id();
    const int ut = blockIdx.x, rg = blockIdx.y, ks = blockIdx.z;
    const int unit = ut * 16 + (lane & 15);
    const int kq = (lane >> 4) * 8;  // MFMA operand layout: lane l supplies row/column
                                     // l % 16 with K values 8 * (l / 16) .. + 8
    const size_t H3 = (size_t)3 * a.H;
    const bf16_t* xrow[kRowBlocks];
    const bf16_t* hrow[kRowBlocks];
    bool xok[kRowBlocks];
#pragma unroll
    for (int rb = 0; rb < kRowBlocks; ++rb) {
        const int r = rg * 64 + rb * 16 + (lane & 15);
        int xr = -1;
        if (r < a.B) xr = a.xtok ? a.xtok[r] : r;
        xok[rb] = xr >= 0;  // rows past B and idle rows contribute zeros
        xrow[rb] = (const bf16_t*)a.x + (size_t)(xok[rb] ? xr : 0) * a.E;
        hrow[rb] = a.hsplit + (xok[rb] ? state_index(a, r) * H3 : 0);
    }
    const bf16_t* wi = (const bf16_t*)a.W_ih + (size_t)unit * a.E;
    const bf16_t* wh = (const bf16_t*)a.W_hh + (size_t)unit * a.H;
    const size_t gi = (size_t)a.H * a.E, gh = (size_t)a.H * a.H;

    f32x4 acc[kRowBlocks][4];
#pragma unroll
    for (int rb = 0; rb < kRowBlocks; ++rb)
#pragma unroll
        for (int g = 0; g < 4; ++g) acc[rb][g] = f32x4{0.f, 0.f, 0.f, 0.f};

    const int nE = a.E / 32, nK = nE + a.H / 32;
    const int c0 = ks * nK / a.ksplit, c1 = (ks + 1) * nK / a.ksplit;
    const int w0 = c0 + wave * (c1 - c0) / 4, w1 = c0 + (wave + 1) * (c1 - c0) / 4;
    const bf16x8 zero = __builtin_bit_cast(bf16x8, u32x4{0u, 0u, 0u, 0u});

#pragma unroll 2
    for (int c = w0; c < min(w1, nE); ++c) {
        const int k = c * 32 + kq;
        const bf16x8 br = load_bf16x8(wi + k);
        const bf16x8 bz = load_bf16x8(wi + gi + k);
        const bf16x8 bn = load_bf16x8(wi + 2 * gi + k);
        bf16x8 av[kRowBlocks];
#pragma unroll
        for (int rb = 0; rb < kRowBlocks; ++rb) av[rb] = xok[rb] ? load_bf16x8(xrow[rb] + k) : zero;
#pragma unroll
        for (int rb = 0; rb < kRowBlocks; ++rb) {
            acc[rb][0] = mfma(av[rb], br, acc[rb][0]);
            acc[rb][1] = mfma(av[rb], bz, acc[rb][1]);
            acc[rb][2] = mfma(av[rb], bn, acc[rb][2]);
        }
    }
#pragma unroll 2
    for (int c = max(w0, nE); c < w1; ++c) {
        const int k = (c - nE) * 32 + kq;
        const bf16x8 br = load_bf16x8(wh + k);
        const bf16x8 bz = load_bf16x8(wh + gh + k);
        const bf16x8 bn = load_bf16x8(wh + 2 * gh + k);
        bf16x8 p[kRowBlocks][3];
#pragma unroll
        for (int rb = 0; rb < kRowBlocks; ++rb)
#pragma unroll
            for (int s = 0; s < 3; ++s) p[rb][s] = xok[rb] ? load_bf16x8(hrow[rb] + s * a.H + k) : zero;
#pragma unroll
        for (int rb = 0; rb < kRowBlocks; ++rb)
#pragma unroll
            for (int s = 0; s < 3; ++s) {
                acc[rb][0] = mfma(p[rb][s], br, acc[rb][0]);
                acc[rb][1] = mfma(p[rb][s], bz, acc[rb][1]);
                acc[rb][3] = mfma(p[rb][s], bn, acc[rb][3]);
            }
    }

    // the four waves' sums meet in wave 0, added in wave order
    if (wave > 0) {
#pragma unroll
        for (int rb = 0; rb < kRowBlocks; ++rb)
#pragma unroll
            for (int g = 0; g < 4; ++g)
#pragma unroll
                for (int e = 0; e < 4; ++e) red[wave - 1][(rb * 4 + g) * 4 + e][lane] = acc[rb][g][e];
    }
    __syncthreads();
    if (wave != 0) return;
#pragma unroll
    for (int rb = 0; rb < kRowBlocks; ++rb)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            // lane holds row rg*64 + rb*16 + (lane/16)*4 + e of hidden unit `unit`
            const int row = rg * 64 + rb * 16 + (lane >> 4) * 4 + e;
            if (row >= a.B) continue;
            float* out = a.partial + ((size_t)(ks * a.B + row) * kGateSlots) * a.H + unit;
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const int i = (rb * 4 + g) * 4 + e;
                out[(size_t)g * a.H] =
                    ((acc[rb][g][e] + red[0][i][lane]) + red[1][i][lane]) + red[2][i][lane];
            }
            if (ks == 0) {  // previous state of (row, unit), rebuilt exactly from its parts
                const int xr = a.xtok ? a.xtok[row] : row;
                float hp = 0.f;
                if (xr >= 0) {
                    const bf16_t* hs = a.hsplit + state_index(a, row) * H3 + unit;
                    hp = (bf16_to_f32(hs[0]) + bf16_to_f32(hs[a.H])) + bf16_to_f32(hs[2 * a.H]);
                }
                out[(size_t)4 * a.H] = hp;
            }
        }
}

// binary32 path (small configurations): one thread per (row, hidden unit),
// plain FMA loops over the full K (single K range).
__global__ __launch_bounds__(64) void gru_gates_f32_kernel(GruGatesArgs a) {
    const int b = blockIdx.y;
    const int j = blockIdx.x * 64 + (int)threadIdx.x;
    if (j >= a.H) return;
    float* out = a.partial + ((size_t)b * kGateSlots) * a.H + j;
    const int xr = a.xtok ? a.xtok[b] : b;
    if (xr < 0) {
        for (int g = 0; g < kGateSlots; ++g) out[(size_t)g * a.H] = 0.f;
        return;
    }
    const float* x = (const float*)a.x + (size_t)xr * a.E;
    const float* h = a.hf + state_index(a, b) * a.H;
    const float* wi = (const float*)a.W_ih;
    const float* wh = (const float*)a.W_hh;
    float ir = 0.f, iz = 0.f, in = 0.f, hr = 0.f, hz = 0.f, hn = 0.f;
    for (int k = 0; k < a.E; ++k) {
        const float xv = x[k];
        ir = fmaf(wi[(size_t)j * a.E + k], xv, ir);
        iz = fmaf(wi[(size_t)(a.H + j) * a.E + k], xv, iz);
        in = fmaf(wi[(size_t)(2 * a.H + j) * a.E + k], xv, in);
    }
    for (int k = 0; k < a.H; ++k) {
        const float hv = h[k];
        hr = fmaf(wh[(size_t)j * a.H + k], hv, hr);
        hz = fmaf(wh[(size_t)(a.H + j) * a.H + k], hv, hz);
        hn = fmaf(wh[(size_t)(2 * a.H + j) * a.H + k], hv, hn);
    }
    out[0] = ir + hr;
    out[(size_t)a.H] = iz + hz;
    out[(size_t)2 * a.H] = in;
    out[(size_t)3 * a.H] = hn;
    out[(size_t)4 * a.H] = h[j];
}

// h [B, H] binary32 -> its exact three-part bf16 split [B, 3, H].
__global__ __launch_bounds__(256) void split_kernel(const float* h, bf16_t* parts, int B, int H) {
    const int b = blockIdx.x;
    for (int k = threadIdx.x; k < H; k += blockDim.x) {
        uint32_t p[3];
        split3_bf16(h[(size_t)b * H + k], p);
        for (int s = 0; s < 3; ++s) parts[((size_t)b * 3 + s) * H + k] = (bf16_t)p[s];
    }
}

// h_out[b] = GRU cell from the K-range partial sums of row b.
__global__ __launch_bounds__(256) void finalize_kernel(const float* partial, int ksplit,
                                                       const void* b_ih, const void* b_hh,
                                                       float* h_out, int B, int H, int dtype) {
    const int b = blockIdx.x;
    for (int k = threadIdx.x; k < H; k += blockDim.x)
        h_out[(size_t)b * H + k] = gru_from_partials(partial, ksplit, B, b, H, k, b_ih, b_hh, dtype);
}

}  // namespace

int gru_ksplit(int B, int E, int H, int dtype) {
    if (dtype != 1) return 1;
    const int nK = (E + H) / 32;
    const int tiles = (H / 16) * ((B + 63) / 64);
    int ks = (256 + tiles - 1) / max(tiles, 1);  // ~one workgroup per CU
    return max(1, min(ks, max(1, nK / 8)));       // >= 2 chunks per wave
}

hipError_t launch_gru_gates(const GruGatesArgs& a, hipStream_t stream) {
    if (a.B == 0) return hipSuccess;
    if (a.dtype == 1) {
        dim3 grid(a.H / 16, (a.B + 63) / 64, a.ksplit);
        gru_gates_bf16_kernel<<<grid, kThreads, 0, stream>>>(a);
    } else {
        dim3 grid((a.H + 63) / 64, a.B, 1);
        gru_gates_f32_kernel<<<grid, 64, 0, stream>>>(a);
    }
    return hipGetLastError();
}

hipError_t launch_split(const float* h, bf16_t* parts, int B, int H, hipStream_t stream) {
    if (B == 0) return hipSuccess;
    split_kernel<<<B, 256, 0, stream>>>(h, parts, B, H);
    return hipGetLastError();
}

hipError_t launch_finalize(const float* partial, int ksplit, const void* b_ih, const void* b_hh,
                           float* h_out, int B, int H, int dtype, hipStream_t stream) {
    if (B == 0) return hipSuccess;
    finalize_kernel<<<B, 256, 0, stream>>>(partial, ksplit, b_ih, b_hh, h_out, B, H, dtype);
    return hipGetLastError();
}

}  // namespace dt
