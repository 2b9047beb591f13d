// dt_launch.h -- host-side launchers of the library's kernels and the
// per-call argument block of the expansion.  Internal; not part of the C ABI.
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace dt {

typedef unsigned long long u64;

// Optional timing of one launch: when `start` is set, the two events take the
// kernel's own begin and end times (hipExtLaunchKernel), so their difference
// is the kernel's duration without the dispatch gap.
struct LaunchEvents {
    hipEvent_t start = nullptr, stop = nullptr;
};
template <typename T> struct same_type { using type = T; };
template <typename... P>
hipError_t launch_kernel(void (*k)(P...), dim3 grid, dim3 block, unsigned shm, hipStream_t s,
                         LaunchEvents ev, typename same_type<P>::type... args) {
    if (!ev.start) {
        hipLaunchKernelGGL(k, grid, block, shm, s, args...);
        return hipGetLastError();
    }
    void* argv[] = {(void*)&args...};
    return hipExtLaunchKernel((const void*)k, grid, block, argv, shm, s, ev.start, ev.stop, 0);
}

// ---- top-M select (topm.hip) ----------------------------------------------
int topm_segments(int rows, int V);
// rows = B*L rows of V logits; partial: rows*nseg*64 keys of scratch.
// ev (optional) times the select kernel alone (not the merge).  With
// tail_out (full-vocabulary mode) tail_out[row] also receives log sum of
// exp(x / T) over the row's logits outside its top M (-inf if none), with
// tail_c = log2(e) / T (T = 1 when T = 0); tail_part is rows*nseg*2 floats
// of scratch.
// side: words that the next kernel on the stream needs zeroed and a clock
// pair it needs set to (max, 0) (the persistent expansion's flags and its
// device-clock span), written by the select's first workgroup beside its row
// so that no launch of their own runs between the two kernels.
struct TopmSide {
    unsigned* zero = nullptr;  // [nzero] (NULL: none)
    int nzero = 0;
    unsigned long long* clock = nullptr;  // [2] (NULL: none)
};
hipError_t launch_topm(const void* base, int dtype, int rows, int V, int nseg, u64* partial, int M,
                       int32_t* idx, float* val, hipStream_t stream, LaunchEvents ev = {},
                       float tail_c = 0.f, float* tail_out = nullptr, float* tail_part = nullptr,
                       TopmSide side = {});

// ---- GRU gate contraction (gru.hip) -----------------------------------------
// bf16 path: the activations come packed for the MFMA operands (see
// pack_index_x / pack_index_h): row b's embedding in `xpack` and the exact
// three-part bf16 split of its previous state in `hpack` (idle rows are
// zero).  binary32 path: row b reads x + xrow(b) * E with xrow(b) = xtok ?
// xtok[b] : b (a negative xtok[b] marks an idle row) and state number
// b * hrows + (hsel ? hsel[b] : 0) of `hf` ([H] per state).  Both write the
// K-range partial sums to `partial` ([ksplit][B][kGateSlots][H], see
// dt_device.h); the consumer supplies the previous state itself.
struct GruGatesArgs {
    const uint16_t* xpack;
    const uint16_t* hpack;
    const void* x;
    const int32_t* xtok;
    const float* hf;
    int hrows;
    const int32_t* hsel;
    const void* W_ih;
    const void* W_hh;
    float* partial;
    int B, E, H, ksplit, dtype;
    int xwaves;  // bf16 path: waves per workgroup on the x part (set by the launcher)
    // bf16 path: the weights in MFMA operand tiles ([H/16][3][nE + nH][512],
    // see pack_index_w).  wmode 0: read W_ih / W_hh; 1: read them and write
    // this copy; 2: read this copy.
    uint16_t* wpack;
    int wmode;
};
// Packed activations (bf16 elements).  Rows are grouped in blocks of 16 (the
// MFMA operand rows); a block's K range is cut into 32-wide chunks; one chunk
// of one block is 16 rows x 32 elements = 1 KB, contiguous, so a wave loads an
// operand tile with one contiguous 1 KB read.  Row blocks are allocated for
// B rounded up to 64 rows.
__host__ __device__ inline size_t pack_index_x(int b, int k, int E) {
    return ((size_t)((b >> 4) * (E >> 5) + (k >> 5)) * 16 + (b & 15)) * 32 + (k & 31);
}
__host__ __device__ inline size_t pack_index_h(int b, int part, int k, int H) {
    return ((size_t)(((b >> 4) * 3 + part) * (H >> 5) + (k >> 5)) * 16 + (b & 15)) * 32 + (k & 31);
}
inline int pack_rows(int B) { return (B + 63) / 64 * 64; }
// Packed weights: operand tile (unit tile ut of 16 hidden units, gate g, K
// chunk c of nchunk = E/32 + H/32; x chunks first) is 512 contiguous bf16,
// lane l's 8 elements (unit l % 16, K 8 * (l / 16) .. + 8 of the chunk) at l * 8.
__host__ __device__ inline size_t pack_index_w(int ut, int g, int c, int nchunk) {
    return ((size_t)(ut * 3 + g) * nchunk + c) * 512;
}
__device__ __forceinline__ size_t state_index(const GruGatesArgs& a, int b) {
    return (size_t)b * a.hrows + (size_t)(a.hsel ? a.hsel[b] : 0);
}
int gru_ksplit(int B, int E, int H, int dtype);
constexpr int kGateSlotsHost = 4;  // == kGateSlots (dt_device.h)
hipError_t launch_gru_gates(const GruGatesArgs& a, hipStream_t stream, LaunchEvents ev = {});
// x [B, E] bf16 and h [B, H] binary32 -> packed activations (rows B .. pack_rows(B) zero)
hipError_t launch_pack(const uint16_t* x, const float* h, uint16_t* xpack, uint16_t* hpack, int B, int E,
                       int H, hipStream_t stream);
// h_out [B, H] from the partial sums and the previous state h [B, H]
hipError_t launch_finalize(const float* partial, int ksplit, const void* b_ih, const void* b_hh,
                           const float* h, float* h_out, int B, int H, int dtype, hipStream_t stream);

// ---- expansion (expand.hip) -------------------------------------------------
constexpr int kStateWords = 8;
struct NodeArgs {
    // problem
    int B, L, V, E, H, M, n, dtype;
    int marginal;  // 1: factorized scores (no GRU, no correction)
    float temp;  // T > 0 divides the corrected logits; 0 = unscaled
    float eps;
    // inputs
    const void* C;
    const float* h0;
    const int32_t* tidx;  // [B, L, M] top-M tables
    const float* tval;
    // workspace
    const void* b_ih;
    const void* b_hh;
    float* hstate;       // [B, n+1, H] hidden state per tree slot (binary32)
    uint16_t* hsplit;    // [B, n+1, 3, H] its exact bf16 parts (bf16 path)
    const float* partial;  // gate partial sums of the preceding contraction
    int ksplit;
    int32_t* gru_tok;    // [B] token of the slot to advance next, -1 = idle row
    int32_t* gru_par;    // [B] its parent slot (whose state is advanced)
    int32_t* child_tok;  // [B, n+1, 64] sorted children per slot
    float* child_lp;     // [B, n+1, 64]
    u64* ckey;           // [B, n+1, 64] unsorted child keys, sorted by the next step
    u64* queue;          // [B, 64] candidate keys, 0 = empty
    int32_t* rstate;     // [B, kStateWords] per-request state left for the next step:
                         // count, next GRU token, queue size, flags, depth of the next slot
    int32_t* nidx;       // [B, 64] candidate tokens of the slot expanded next
    float* nval;         // [B, 64] their base logits
    const void* emb;     // [V, E] token embeddings
    uint16_t* xpack;     // packed activations of the next contraction (bf16 path; see
    uint16_t* hpack;     // pack_index_x / pack_index_h), NULL on the binary32 path
    float* hprev;        // [B, H] the next expanded slot's parent state (bf16 path), or NULL
    const float* tail;   // [B, L] full-vocabulary mode: each row's tail_lse; NULL = M-slice softmax
    const float* table;  // [V, 3H] folded input projection (b_ih + W_ih . Emb[v]); NULL = contracted
    // outputs
    int32_t* tokens;
    int32_t* parents;
    int32_t* depths;
    float* scores;
    uint8_t* mask;
    int32_t* count;
    uint32_t* flags;
};
// Word offsets of the node kernel's dynamic LDS arrays.
struct NodeLds {
    size_t hs, zs, sc, par, tidx, tval, ctok, clp;
    size_t bytes;
};
NodeLds node_lds_plan(int L, int M, int n, int H);
// One expansion step of the standard or folded path (not the factorized mode).
hipError_t launch_node_step(const NodeArgs& a, const NodeLds& lp, int step, hipStream_t stream,
                            LaunchEvents ev = {});
// The factorized mode (a.marginal) expanded in one launch: steps 0 .. n-1 of
// every request, one workgroup per request looping over them.
hipError_t launch_marginal_build(const NodeArgs& a, const NodeLds& lp, hipStream_t stream, LaunchEvents ev = {});

// ---- fused pipelined expansion (expand.hip, bf16) ----------------------------
// One launch per expansion step runs two kinds of workgroups side by side:
// `ng` contraction workgroups (16 hidden units x one of `ksplit` K ranges
// each) and one node workgroup per request.  The contraction of launch t
// takes, per request, an x row (the embedding of the token whose input
// projection the request needs next: a prediction of its next expansion, or
// the node it has to expand) and an h row (the state of the node it expanded
// at launch t - 1), so the node workgroups of launch t expand with what
// launch t - 1 contracted.  See expand.hip.
struct PipeArgs {
    int B, L, V, E, H, M, n;
    int T;                // launches per call
    int ng;               // contraction workgroups (blocks 0 .. ng - 1)
    int ksx, ksh;         // partial sums of a gate's x part, of its h part
    float temp, eps;
    const void* C;
    const float* h0;
    const int32_t* tidx;  // [B, L, M] top-M tables
    const float* tval;
    const float* tail;    // [B, L] full-vocabulary mode, or NULL
    const void* emb;
    const void* W_ih;
    const void* W_hh;
    const void* b_ih;
    const void* b_hh;
    // workspace
    uint16_t* xpack[2];   // contraction activations by launch parity (pack_index_x / _h)
    uint16_t* hpack[2];
    int32_t* xtok[2];     // [B] token of launch t's x row (parity t & 1), -1 = none
    int32_t* hslot[2];    // [B] slot whose state is launch t's h row, -1 = none
    float* gi;            // [2][ksx][B][3][H] x-part gate sums by launch parity
    float* gh;            // [B][n+1][ksh][3][H] h-part gate sums per slot
    float* hstate;        // [B][n+1][H] binary32 state per slot (slot 0 = h0)
    int32_t* exp_at;      // [B][n+1] launch that expanded the slot
    unsigned* done;       // [T] contraction workgroups finished, per launch
    unsigned* gflag;      // [ng] persistent launch: last step each contraction workgroup finished
    unsigned* hflag;      // [2][B] persistent launch: step and h-row slot per node workgroup (hflag_word)
    unsigned* xflag;      // [2][B] persistent launch: x token, wait bit and step per node workgroup
    unsigned* perr;       // a wait of the persistent launch ran out (nonzero)
    unsigned long long* tclock;  // [2] persistent launch: device clock at its first workgroup's start and
                                 // its last one's end (min / max; NULL: not timed)
    int32_t* active;      // [2][T] launch t's contraction has a row; some request waits for it
    uint16_t* wpack;      // the weights in operand tiles (written by launch 0)
    int32_t* child_tok;   // [B, n+1, 64]
    float* child_lp;
    u64* ckey;            // [B, n+1, 64] unsorted child keys
    u64* queue;           // [B, 64]
    int32_t* rstate;      // [B, kStateWords]
    int32_t* nidx;        // [B, 64] candidates of the slot to expand
    float* nval;
    // outputs
    int32_t* tokens;
    int32_t* parents;
    int32_t* depths;
    float* scores;
    uint8_t* mask;
    int32_t* count;
    uint32_t* flags;
};
// Launch geometry of the fused expansion for a configuration, or ng = 0 when
// it does not apply (binary32, the factorized mode, too many requests).
struct PipePlan {
    int ng, ksx, ksh, rb;
    size_t lds;  // dynamic LDS bytes
};
PipePlan pipe_plan(int B, int L, int E, int H, int M, int n);
hipError_t launch_pipe_step(const PipeArgs& a, const PipePlan& pp, const NodeLds& lp, int t, hipStream_t stream,
                            LaunchEvents ev = {});
// The same expansion as one cooperative launch of the same grid: every step of
// the call, the workgroups kept resident and handing over through counters
// (see expand.hip).  pers_supported: the device can hold the whole grid at
// once, V is small enough for a token in a flag word and V E for a 32-bit
// row offset (checked once per plan); launch_pers_build launches it.  The
// call's flags, the pers_flag_words(pp, B) words from a.gflag on, must be
// zero when it starts, and its clock pair (when timed) at (max, 0): the
// top-M select before it sets them (TopmSide).
// More requests than one grid holds (B > kPipeSliceB) run as consecutive
// launches of kPipeSliceB requests each (the last one takes the rest), every
// launch with its own run of flag words; the plan is that of kPipeSliceB.
constexpr int kPipeSliceB = 64;
bool pers_supported(const PipePlan& pp, int B, int V, int E);
inline int pers_flag_words(const PipePlan& pp, int B) { return pp.ng + 6 * B + 1; }
inline int pers_slices(int B) { return (B + kPipeSliceB - 1) / kPipeSliceB; }
inline int pers_slice_b(int B) { return B < kPipeSliceB ? B : kPipeSliceB; }
// coop: a cooperative launch (the runtime guarantees the grid's
// co-residency); otherwise a plain launch of the same grid, resident by the
// occupancy check alone (every wait is bounded either way).
hipError_t launch_pers_build(const PipeArgs& a, const PipePlan& pp, const NodeLds& lp, hipStream_t stream,
                             LaunchEvents ev = {}, bool coop = true);

// Conditional children distribution of one node per row (dt_correct).
hipError_t launch_correct(const int32_t* tidx, const float* tval, const void* C, const float* h,
                          const int32_t* pos, int32_t* tok_sorted, float* lp_sorted, int B, int L,
                          int H, int M, int dtype, float temp, hipStream_t stream);

// ---- folded input projection (fold.hip) ---------------------------------------
// table [V, 3H] binary32 = b_ih + W_ih . Emb[v] for every token v
hipError_t launch_fold(const void* emb, const void* W_ih, const void* b_ih, float* table, int V, int E, int H,
                       int dtype, hipStream_t stream);

// ---- greedy acceptance walk (accept.hip) --------------------------------------
// trees [B, n+1] as dt_build writes them, target [B, n+1] -> path [B, n+1],
// accepted [B], bonus [B]
hipError_t launch_accept_greedy(const int32_t* tokens, const int32_t* parents, const int32_t* count,
                                const int32_t* target, int B, int n, int32_t* path, int32_t* accepted,
                                int32_t* bonus, hipStream_t stream, LaunchEvents ev = {});

}  // namespace dt
