// dt_launch.h -- host-side launchers of the library's kernels and the
// per-call argument block of the expansion.  Internal; not part of the C ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace dt {

typedef unsigned long long u64;

// ---- top-M select (topm.hip) ----------------------------------------------
int topm_segments(int rows, int V);
// rows = B*L rows of V logits; partial: rows*nseg*64 keys of scratch.
// ev_mid (optional) is recorded between the select and the merge kernel.
hipError_t launch_topm(const void* base, int dtype, int rows, int V, int nseg, u64* partial, int M,
                       int32_t* idx, float* val, hipStream_t stream, hipEvent_t ev_mid);

// ---- GRU gate contraction (gru.hip) ----------------------------------------
// Partial gate sums for every row b < B, written as
//   gates[((s * B + b) * 4 + g) * H + j],  g = 0 reset, 1 update, 2 new (x
// part), 3 new (h part), s < ksplit (K-split slices, summed by the consumer).
// Row b's GRU input x is x + xrow(b) * E with xrow(b) = xtok ? xtok[b] : b;
// a negative xtok[b] marks an idle row (its gates are not needed).  Row b's
// hidden state is h + b * hstride + (hsel ? hsel[b] : 0) * H.
struct GruGemmArgs {
    const void* x;
    const int32_t* xtok;
    const float* h;
    const int32_t* hsel;
    size_t hstride;
    const void* W_ih;
    const void* W_hh;
    float* gates;
    int B, E, H, ksplit, dtype;
};
int gru_ksplit(int B, int E, int H, int dtype);
hipError_t launch_gru_gemm(const GruGemmArgs& a, hipStream_t stream);
// h_out[b] = GRU elementwise update from the gate sums, biases and h[b].
hipError_t launch_gru_finalize(const float* gates, int ksplit, const void* b_ih, const void* b_hh,
                               const float* h, float* h_out, int B, int H, int dtype,
                               hipStream_t stream);

// ---- expansion (expand.hip) -------------------------------------------------
struct NodeArgs {
    // problem
    int B, L, V, E, H, M, n, dtype;
    float temp;  // T > 0 divides the corrected logits; 0 = unscaled
    float eps;
    // inputs
    const void* C;
    const void* b_ih;
    const void* b_hh;
    const float* h0;
    const int32_t* tidx;  // [B, L, M] top-M tables
    const float* tval;
    // workspace
    float* hstate;       // [B, n+1, H] hidden state per tree slot
    float* gates;        // GRU partial gate sums (see GruGemmArgs)
    int ksplit;
    int32_t* gru_tok;    // [B] token to feed, -1 = idle row
    int32_t* gru_par;    // [B] parent slot whose state is advanced
    int32_t* child_tok;  // [B, n+1, 64] sorted children per slot
    float* child_lp;     // [B, n+1, 64]
    u64* queue;          // [B, 64] candidate keys, 0 = empty
    int32_t* qsize;      // [B]
    // outputs
    int32_t* tokens;
    int32_t* parents;
    int32_t* depths;
    float* scores;
    uint8_t* mask;
    int32_t* count;
    uint32_t* flags;
};
hipError_t launch_node_step(const NodeArgs& a, int step, hipStream_t stream);

// Conditional children distribution of one node per row (dt_correct).
hipError_t launch_correct(const int32_t* tidx, const float* tval, const void* C, const float* h,
                          const int32_t* pos, int32_t* tok_sorted, float* lp_sorted, int B, int L,
                          int H, int M, int dtype, float temp, hipStream_t stream);

}  // namespace dt
