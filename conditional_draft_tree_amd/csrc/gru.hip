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
// owns 16 hidden units x 64 rows x one of `ksplit` K ranges; its eight waves
// take disjoint chunk ranges over all 64 rows, so every weight element is
// loaded by exactly one wave.  The waves' sums meet in LDS in wave order and
// the workgroup writes its K-range partial sums; the consumer (the node step,
// or gru_finalize) adds the `ksplit` partials in K order and applies the GRU
// cell.  The binary32 state h is fed as the exact sum of three bf16 parts
// (computed once per state by its producer), so the recurrent product is not
// quantized.  The K-range-0 workgroups also copy the previous state into the
// partial buffer, so the consumer needs no dependent load.
#include "dt_device.h"
#include "dt_launch.h"
#include "gate_tile.h"

namespace dt {

namespace {

using gate::bf16x8;
using gate::f32x4;
using gate::u32x4;
using gate::kWaves8;
using gate::row_blocks;
using gate::x_waves;
using gate::kMaxXChunks;
using gate::kMaxHChunks;

// WM: weight source (0: W_ih / W_hh; 1: those, and write the packed copy; 2:
// the packed copy), a template parameter so that each variant keeps one
// address path and no dead store code.  RB: 16-row blocks per workgroup.
template <int WM, int RB>
__global__ __launch_bounds__(kWaves8 * 64) void gru_gates_bf16_kernel(GruGatesArgs a) {
    // every wave's sums of the workgroup's (RB x 16) x 16 outputs x 4 gates
    // (128 KB at RB = 4)
    __shared__ f32x4 red[kWaves8][RB * 4][kWave];
    const int wave = threadIdx.x / kWave, lane = lane_id();
    const int ut = blockIdx.x, rg = blockIdx.y, ks = blockIdx.z;
    f32x4 acc[RB][4];
    gate::tile_accumulate<WM, RB>(a, ut, rg, ks, acc);

    // the 8 waves' sums added in wave order (one LDS round trip); all 512
    // threads write the workgroup's partial sums
#pragma unroll
    for (int rb = 0; rb < RB; ++rb)
#pragma unroll
        for (int g = 0; g < 4; ++g) red[wave][rb * 4 + g][lane] = acc[rb][g];
    __syncthreads();
#pragma unroll
    for (int h2 = 0; h2 < 2; ++h2) {
        const int idx = (int)threadIdx.x + h2 * kWaves8 * kWave;  // (rb, g, lane) of RB x 4 x 64
        if (idx >= RB * 4 * kWave) break;
        const int sl = idx >> 6, ln = idx & 63;
        f32x4 sum = red[0][sl][ln];
#pragma unroll
        for (int w2 = 1; w2 < kWaves8; ++w2) sum += red[w2][sl][ln];
        const int rb = sl >> 2, g = sl & 3;
#pragma unroll
        for (int e = 0; e < 4; ++e) {  // MFMA output rows 4 * (lane / 16) + e
            const int row = rg * 64 + rb * 16 + (ln >> 4) * 4 + e;
            if (row < a.B)
                a.partial[((size_t)(ks * a.B + row) * kGateSlots + g) * a.H + ut * 16 + (ln & 15)] = sum[e];
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
}

// x [B, E] bf16 and h [B, H] binary32 -> packed activations; rows B .. of the
// last 64-row group are zero.
__global__ __launch_bounds__(256) void pack_kernel(const bf16_t* x, const float* h, bf16_t* xpack,
                                                   bf16_t* hpack, int B, int E, int H) {
    const int b = blockIdx.x;
    const bool in = b < B;
    for (int k = threadIdx.x; k < E; k += blockDim.x)
        xpack[pack_index_x(b, k, E)] = in ? x[(size_t)b * E + k] : (bf16_t)0;
    for (int k = threadIdx.x; k < H; k += blockDim.x) {
        uint32_t p[3] = {0u, 0u, 0u};
        if (in) split3_bf16(h[(size_t)b * H + k], p);
        for (int s = 0; s < 3; ++s) hpack[pack_index_h(b, s, k, H)] = (bf16_t)p[s];
    }
}

// h_out[b] = GRU cell from the K-range partial sums of row b and its state h[b].
__global__ __launch_bounds__(256) void finalize_kernel(const float* partial, int ksplit,
                                                       const void* b_ih, const void* b_hh, const float* h,
                                                       float* h_out, int B, int H, int dtype) {
    const int b = blockIdx.x;
    for (int k = threadIdx.x; k < H; k += blockDim.x)
        h_out[(size_t)b * H + k] =
            gru_from_partials(partial, ksplit, B, b, H, k, b_ih, b_hh, dtype, h[(size_t)b * H + k]);
}

}  // namespace

int gru_ksplit(int B, int E, int H, int dtype) {
    if (dtype != 1) return 1;
    // ~one workgroup per CU, and a single load batch per wave where possible
    const int nE = E / 32, nH = H / 32, rb = row_blocks(B);
    const int tiles = (H / 16) * ((B + 63) / 64);
    int best = kMaxKsplit;
    for (int ks = 1; ks <= kMaxKsplit; ++ks) {
        const int wx = x_waves(nE, nH, ks, rb), nx = ks * wx, nh = ks * (kWaves8 - wx);
        const int xmax = nE ? (nE + nx - 1) / nx : 0, hmax = nH ? (nH + nh - 1) / nh : 0;
        if (xmax <= kMaxXChunks && hmax <= kMaxHChunks && tiles * ks >= 192) return ks;
        if (xmax <= kMaxXChunks && hmax <= kMaxHChunks) best = min(best, ks);
    }
    return best;
}

hipError_t launch_gru_gates(const GruGatesArgs& a, hipStream_t stream, LaunchEvents ev) {
    if (a.B == 0) return hipSuccess;
    if (a.dtype == 1) {
        GruGatesArgs b = a;
        const int rb = row_blocks(a.B);
        b.xwaves = x_waves(a.E / 32, a.H / 32, a.ksplit, rb);
        const dim3 grid(a.H / 16, (a.B + 63) / 64, a.ksplit), block(kWaves8 * kWave);
        const int wm = a.wpack ? (a.wmode == 2 ? 2 : a.wmode == 1 ? 1 : 0) : 0;
#define DT_GATES(WM, RB) \
    if (wm == WM && rb == RB) return launch_kernel(gru_gates_bf16_kernel<WM, RB>, grid, block, 0, stream, ev, b);
        DT_GATES(2, 4) DT_GATES(1, 4) DT_GATES(0, 4) DT_GATES(2, 2) DT_GATES(1, 2) DT_GATES(0, 2)
        DT_GATES(2, 1) DT_GATES(1, 1) DT_GATES(0, 1)
#undef DT_GATES
        return hipErrorInvalidValue;
    }
    return launch_kernel(gru_gates_f32_kernel, dim3((a.H + 63) / 64, a.B, 1), dim3(64), 0, stream, ev, a);
}

hipError_t launch_pack(const uint16_t* x, const float* h, uint16_t* xpack, uint16_t* hpack, int B, int E,
                       int H, hipStream_t stream) {
    if (B == 0) return hipSuccess;
    pack_kernel<<<pack_rows(B), 256, 0, stream>>>((const bf16_t*)x, h, (bf16_t*)xpack, (bf16_t*)hpack, B, E, H);
    return hipGetLastError();
}

hipError_t launch_finalize(const float* partial, int ksplit, const void* b_ih, const void* b_hh,
                           const float* h, float* h_out, int B, int H, int dtype, hipStream_t stream) {
    if (B == 0) return hipSuccess;
    finalize_kernel<<<B, 256, 0, stream>>>(partial, ksplit, b_ih, b_hh, h, h_out, B, H, dtype);
    return hipGetLastError();
}

}  // namespace dt
