// fold.hip -- the GRU's input projection of every vocabulary token, once per
// model: table[v][j] = b_ih[j] + sum_k W_ih[j][k] * Emb[v][k], binary32.
//
// A node's GRU input is the embedding of its own token ([captcha]
// "Methodology -- deep read": the GRU state is advanced along the path with
// the realized tokens), so W_ih . x + b_ih takes one of V values, fixed by
// the model.  With this table a step's gate contraction only needs the
// recurrent part W_hh . h, and the node step adds the popped token's row:
// 3H floats per request instead of an E-wide contraction per step.
#include "dt_device.h"
#include "dt_launch.h"

namespace dt {

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

constexpr int kFoldChunks = 4;  // 32-wide K chunks per load batch

__device__ __forceinline__ bf16x8 ld8(const bf16_t* p) {
    return __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(p));
}

// Tiles of 64 tokens x 64 outputs, 4 waves: wave w takes tokens 16w .. 16w+15
// of the tile and all 64 outputs (4 MFMA column blocks); the token rows are
// the A operand and the W_ih rows the B operand of v_mfma_f32_16x16x32_bf16
// (lane l supplies row / column l % 16 with K values 8 (l / 16) .. + 8).
// Rows past V or N read the last row; their results are not stored.
__global__ __launch_bounds__(256) void fold_bf16_kernel(const bf16_t* __restrict__ emb,
                                                        const bf16_t* __restrict__ W,
                                                        const bf16_t* __restrict__ bias,
                                                        float* __restrict__ table, int V, int E, int N) {
    const int wave = threadIdx.x / kWave, lane = lane_id();
    const int v0 = blockIdx.x * 64 + wave * 16, j0 = blockIdx.y * 64;
    const int kq = (lane >> 4) * 8;
    const bf16_t* arow = emb + (size_t)min(v0 + (lane & 15), V - 1) * E + kq;
    const bf16_t* brow[4];
#pragma unroll
    for (int cb = 0; cb < 4; ++cb) brow[cb] = W + (size_t)min(j0 + cb * 16 + (lane & 15), N - 1) * E + kq;
    const bf16x8 zero = __builtin_bit_cast(bf16x8, u32x4{0u, 0u, 0u, 0u});
    f32x4 acc[4];
#pragma unroll
    for (int cb = 0; cb < 4; ++cb) acc[cb] = f32x4{0.f, 0.f, 0.f, 0.f};
    const int nc = E / 32;
    for (int c0 = 0; c0 < nc; c0 += kFoldChunks) {
        bf16x8 av[kFoldChunks], bv[kFoldChunks][4];
#pragma unroll
        for (int i = 0; i < kFoldChunks; ++i) {
            const int c = min(c0 + i, nc - 1);  // chunks past nc: zero A operand
            const bf16x8 x = ld8(arow + (size_t)c * 32);
            av[i] = c0 + i < nc ? x : zero;
#pragma unroll
            for (int cb = 0; cb < 4; ++cb) bv[i][cb] = ld8(brow[cb] + (size_t)c * 32);
        }
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int i = 0; i < kFoldChunks; ++i)
#pragma unroll
            for (int cb = 0; cb < 4; ++cb)
                acc[cb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av[i], bv[i][cb], acc[cb], 0, 0, 0);
    }
#pragma unroll
    for (int cb = 0; cb < 4; ++cb) {
        const int j = j0 + cb * 16 + (lane & 15);
        if (j >= N) continue;
        const float bj = bias ? bf16_to_f32(bias[j]) : 0.f;
#pragma unroll
        for (int e = 0; e < 4; ++e) {  // MFMA output rows 4 (l / 16) + e
            const int v = v0 + (lane >> 4) * 4 + e;
            if (v < V) table[(size_t)v * N + j] = acc[cb][e] + bj;
        }
    }
}

// binary32 inputs (small configurations): one thread per (token, output);
// tokens along the grid's x dimension, whose extent is not limited to 16 bits.
__global__ __launch_bounds__(64) void fold_f32_kernel(const float* __restrict__ emb, const float* __restrict__ W,
                                                      const float* __restrict__ bias, float* __restrict__ table,
                                                      int V, int E, int N) {
    const int v = blockIdx.x, j = blockIdx.y * 64 + (int)threadIdx.x;
    if (j >= N) return;
    float s = bias ? bias[j] : 0.f;
    for (int k = 0; k < E; ++k) s = fmaf(W[(size_t)j * E + k], emb[(size_t)v * E + k], s);
    table[(size_t)v * N + j] = s;
}

}  // namespace

hipError_t launch_fold(const void* emb, const void* W_ih, const void* b_ih, float* table, int V, int E, int H,
                       int dtype, hipStream_t stream) {
    if (V == 0) return hipSuccess;
    const int N = 3 * H;
    if (dtype == 1)
        return launch_kernel(fold_bf16_kernel, dim3((V + 63) / 64, (N + 63) / 64), dim3(256), 0, stream,
                             LaunchEvents{}, (const bf16_t*)emb, (const bf16_t*)W_ih, (const bf16_t*)b_ih, table,
                             V, E, N);
    return launch_kernel(fold_f32_kernel, dim3(V, (N + 63) / 64), dim3(64), 0, stream, LaunchEvents{},
                         (const float*)emb, (const float*)W_ih, (const float*)b_ih, table, V, E, N);
}

}  // namespace dt
