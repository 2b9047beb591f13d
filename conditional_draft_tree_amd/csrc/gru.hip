// gru.hip -- the GRU gate contraction of one expansion step, batched over
// the B requests, and the elementwise GRU update.
//
// Expanding a node advances the GRU hidden state along the node's path with
// its realized token ([captcha] "Methodology -- deep read"; [gist] "Composants
// clés": only the light GRU correction is recomputed per node).  Every request
// pops exactly one node per step, so the B updates of a step form one
// contraction [B, E+H] x [E+H, 3H].  The reset and update gates sum the x and
// h parts; the candidate gate keeps them apart (its h part is scaled by the
// reset gate), hence four accumulators per output unit.
//
// bf16 path: v_mfma_f32_16x16x32_bf16 (gfx950), binary32 accumulation.  A
// workgroup owns 16 hidden units x 64 rows (4 waves x 16 rows) x one K slice
// (ksplit slices, summed in a fixed order by the consumer).  The h operand is
// rounded from binary32 to bf16 (nearest even) as it is loaded.
#include "dt_device.h"
#include "dt_launch.h"

namespace dt {

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

constexpr int kGemmThreads = 256;

__device__ __forceinline__ bf16x8 load_bf16x8(const bf16_t* p) {
    u32x4 v = *reinterpret_cast<const u32x4*>(p);
    return __builtin_bit_cast(bf16x8, v);
}

__device__ __forceinline__ bf16x8 round_f32x8(const float* p) {
    const f32x4 a = *reinterpret_cast<const f32x4*>(p);
    const f32x4 b = *reinterpret_cast<const f32x4*>(p + 4);
    u32x4 w;
    w.x = f32_to_bf16_rne(a.x) | (f32_to_bf16_rne(a.y) << 16);
    w.y = f32_to_bf16_rne(a.z) | (f32_to_bf16_rne(a.w) << 16);
    w.z = f32_to_bf16_rne(b.x) | (f32_to_bf16_rne(b.y) << 16);
    w.w = f32_to_bf16_rne(b.z) | (f32_to_bf16_rne(b.w) << 16);
    return __builtin_bit_cast(bf16x8, w);
}

__global__ __launch_bounds__(kGemmThreads) void gru_gemm_bf16_kernel(GruGemmArgs a) {
    const int wave = threadIdx.x / kWave, lane = lane_id();
    const int j0 = blockIdx.x * 16;
    const int rb = blockIdx.y * 64 + wave * 16;  // this wave's 16 rows
    const int s = blockIdx.z;
    if (rb >= a.B) return;  // no workgroup barrier below

    // MFMA operand layout (16x16x32): lane l supplies row (l % 16) of A and
    // column (l % 16) of B, each with the 8 consecutive K values starting at
    // 8 * (l / 16); the result holds rows 4 * (l / 16) + i, column l % 16.
    const int r = rb + (lane & 15);
    const int kq = (lane >> 4) * 8;
    const bool row_ok = r < a.B;
    int xr = -1;
    if (row_ok) xr = a.xtok ? a.xtok[r] : r;
    const bool x_ok = xr >= 0;
    const bf16_t* xrow = (const bf16_t*)a.x + (size_t)(x_ok ? xr : 0) * a.E;
    const float* hrow = a.h + (row_ok ? (size_t)r * a.hstride +
                                            (size_t)(a.hsel ? a.hsel[r] : 0) * a.H
                                      : 0);
    const int unit = j0 + (lane & 15);
    const bf16_t* wi = (const bf16_t*)a.W_ih + (size_t)unit * a.E;
    const bf16_t* wh = (const bf16_t*)a.W_hh + (size_t)unit * a.H;
    const size_t gi = (size_t)a.H * a.E, gh = (size_t)a.H * a.H;

    f32x4 acc_r = {0.f, 0.f, 0.f, 0.f}, acc_z = acc_r, acc_nx = acc_r, acc_nh = acc_r;
    const int nE = a.E / 32, nK = nE + a.H / 32;
    const int c0 = s * nK / a.ksplit, c1 = (s + 1) * nK / a.ksplit;
    const bf16x8 zero = __builtin_bit_cast(bf16x8, u32x4{0u, 0u, 0u, 0u});

#pragma unroll 4
    for (int c = c0; c < min(c1, nE); ++c) {
        const int k = c * 32 + kq;
        bf16x8 av = x_ok ? load_bf16x8(xrow + k) : zero;
        bf16x8 br = load_bf16x8(wi + k);
        bf16x8 bz = load_bf16x8(wi + gi + k);
        bf16x8 bn = load_bf16x8(wi + 2 * gi + k);
        acc_r = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, br, acc_r, 0, 0, 0);
        acc_z = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, bz, acc_z, 0, 0, 0);
        acc_nx = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, bn, acc_nx, 0, 0, 0);
    }
#pragma unroll 4
    for (int c = max(c0, nE); c < c1; ++c) {
        const int k = (c - nE) * 32 + kq;
        bf16x8 av = row_ok ? round_f32x8(hrow + k) : zero;
        bf16x8 br = load_bf16x8(wh + k);
        bf16x8 bz = load_bf16x8(wh + gh + k);
        bf16x8 bn = load_bf16x8(wh + 2 * gh + k);
        acc_r = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, br, acc_r, 0, 0, 0);
        acc_z = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, bz, acc_z, 0, 0, 0);
        acc_nh = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, bn, acc_nh, 0, 0, 0);
    }

#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int row = rb + (lane >> 4) * 4 + i;
        if (row < a.B) {
            float* g = a.gates + ((size_t)(s * a.B + row) * 4) * a.H + unit;
            g[0] = acc_r[i];
            g[a.H] = acc_z[i];
            g[2 * a.H] = acc_nx[i];
            g[3 * a.H] = acc_nh[i];
        }
    }
}

// binary32 path (small configurations): one thread per (row, hidden unit),
// plain FMA loops; single K slice.
__global__ __launch_bounds__(64) void gru_gemm_f32_kernel(GruGemmArgs a) {
    const int b = blockIdx.y;
    const int j = blockIdx.x * 64 + (int)threadIdx.x;
    if (j >= a.H) return;
    const int xr = a.xtok ? a.xtok[b] : b;
    float* g = a.gates + ((size_t)b * 4) * a.H + j;
    if (xr < 0) {
        g[0] = g[a.H] = g[2 * a.H] = g[3 * a.H] = 0.f;
        return;
    }
    const float* x = (const float*)a.x + (size_t)xr * a.E;
    const float* h = a.h + (size_t)b * a.hstride + (size_t)(a.hsel ? a.hsel[b] : 0) * a.H;
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
    g[0] = ir + hr;
    g[a.H] = iz + hz;
    g[2 * a.H] = in;
    g[3 * a.H] = hn;
}

__global__ __launch_bounds__(256) void gru_finalize_kernel(const float* gates, int ksplit,
                                                           const void* b_ih, const void* b_hh,
                                                           const float* h, float* h_out, int B,
                                                           int H, int dtype) {
    const int b = blockIdx.x;
    for (int k = threadIdx.x; k < H; k += blockDim.x)
        h_out[(size_t)b * H + k] =
            gru_unit_update(gates, ksplit, B, b, H, k, b_ih, b_hh, dtype, h[(size_t)b * H + k]);
}

}  // namespace

int gru_ksplit(int B, int E, int H, int dtype) {
    if (dtype != 1) return 1;
    const int nK = (E + H) / 32;
    const int tiles = (H / 16) * ((B + 63) / 64);
    int ks = (512 + tiles - 1) / max(tiles, 1);
    return max(1, min(ks, max(1, nK / 4)));
}

hipError_t launch_gru_gemm(const GruGemmArgs& a, hipStream_t stream) {
    if (a.B == 0) return hipSuccess;
    if (a.dtype == 1) {
        dim3 grid(a.H / 16, (a.B + 63) / 64, a.ksplit);
        gru_gemm_bf16_kernel<<<grid, kGemmThreads, 0, stream>>>(a);
    } else {
        dim3 grid((a.H + 63) / 64, a.B, 1);
        gru_gemm_f32_kernel<<<grid, 64, 0, stream>>>(a);
    }
    return hipGetLastError();
}

hipError_t launch_gru_finalize(const float* gates, int ksplit, const void* b_ih, const void* b_hh,
                               const float* h, float* h_out, int B, int H, int dtype,
                               hipStream_t stream) {
    if (B == 0) return hipSuccess;
    gru_finalize_kernel<<<B, 256, 0, stream>>>(gates, ksplit, b_ih, b_hh, h, h_out, B, H, dtype);
    return hipGetLastError();
}

}  // namespace dt
