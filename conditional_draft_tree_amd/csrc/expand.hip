// expand.hip -- one step of the conditional best-first expansion, for every
// request at once (one workgroup per request).
//
// DDTree's best-first builder with a max-priority queue keyed by the
// cumulative conditional log-prob, run until n nodes or the maximum depth
// ([captcha] "Methodology -- deep read"; [gist] "Composants clés -- Tas de
// recherche de premier choix à score conditionnel").  Node v's children are
// scored by Domino's correction restricted to the top-M candidates of block
// position depth(v): the gathered rows of the correction matrix times the
// GRU state, added to the gathered base logits ([captcha] "Methodology --
// deep read"), normalized by a log-softmax over the M-slice.
//
// Step s (s = 0 .. n-1) of request b:
//   1. slot s's hidden state (written by the preceding GRU step; the root
//      takes h0), the top-M table, the sorted children of slots < s and the
//      tree so far are loaded into LDS in one round trip;
//   2. slot s's children: z_j = val_j + C[idx_j] . h, z /= T, log-softmax,
//      bitonic sort by (log-prob desc, token asc) across one wave;
//   3. push slot s's best child; pop the best candidate as slot s+1 and push
//      its next-ranked sibling (lazy sibling push: the queue then holds at
//      most n entries, one per lane of a wave);
//   4. stage slot s+1 for the next GRU step;
//   5. after the last step, emit the ancestor-only mask.
// Queue key: (score desc, depth asc, parent slot asc, rank asc).
#include <algorithm>

#include "dt_device.h"
#include "dt_launch.h"
#include "gate_tile.h"

namespace dt {

namespace {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef int i32x4 __attribute__((ext_vector_type(4)));

// dt_correct's kernel: 4 waves, 16 gathered rows each
constexpr int kCorrThreads = 256;
constexpr int kCorrRows = kMaxM / (kCorrThreads / kWave);  // 16

// Threads of the node kernel: 16 waves for the conditional step (its 64
// gathered rows and its state spread over 16 waves, so that a wave waits for
// 4 rows, not 16: the gathers land about twice as fast), 4 for the
// factorized step (no state, no gathers).
template <bool MARG> constexpr int node_threads() { return MARG ? 256 : 1024; }

// Four consecutive elements as binary32.
template <typename T> __device__ __forceinline__ f32x4 load4(const T* p);
template <> __device__ __forceinline__ f32x4 load4<float>(const float* p) {
    return *reinterpret_cast<const f32x4*>(p);
}
template <> __device__ __forceinline__ f32x4 load4<bf16_t>(const bf16_t* p) {
    const uint2 w = *reinterpret_cast<const uint2*>(p);
    return f32x4{__uint_as_float(w.x << 16), __uint_as_float(w.x & 0xFFFF0000u),
                 __uint_as_float(w.y << 16), __uint_as_float(w.y & 0xFFFF0000u)};
}

// One element as binary32.
template <typename T> __device__ __forceinline__ float load1(const T* p);
template <> __device__ __forceinline__ float load1<float>(const float* p) { return *p; }
template <> __device__ __forceinline__ float load1<bf16_t>(const bf16_t* p) {
    return __uint_as_float((uint32_t)*p << 16);
}

template <typename T> struct Row;
template <> struct Row<float> {
    static constexpr int kPerVec = 4;
    __device__ static float dot(const u32x4& v, const float* h) {
        float a = __uint_as_float(v.x) * h[0];
        a = fmaf(__uint_as_float(v.y), h[1], a);
        a = fmaf(__uint_as_float(v.z), h[2], a);
        return fmaf(__uint_as_float(v.w), h[3], a);
    }
};
template <> struct Row<bf16_t> {
    static constexpr int kPerVec = 8;
    __device__ static float dot(const u32x4& v, const float* h) {
        float a = __uint_as_float(v.x << 16) * h[0];
        a = fmaf(__uint_as_float(v.x & 0xFFFF0000u), h[1], a);
        a = fmaf(__uint_as_float(v.y << 16), h[2], a);
        a = fmaf(__uint_as_float(v.y & 0xFFFF0000u), h[3], a);
        a = fmaf(__uint_as_float(v.z << 16), h[4], a);
        a = fmaf(__uint_as_float(v.z & 0xFFFF0000u), h[5], a);
        a = fmaf(__uint_as_float(v.w << 16), h[6], a);
        return fmaf(__uint_as_float(v.w & 0xFFFF0000u), h[7], a);
    }
};

// z[j] = val[j] + C[idx[j]] . h for j < M (all four waves; 16 rows each).
// h is in LDS; z goes to LDS.  Two K chunks of all 16 rows are in flight per
// lane (H = 1024 bf16 rows are covered in one round trip).
template <typename T>
__device__ __forceinline__ void correction_logits(const T* __restrict__ C, const int32_t* idx, const float* val,
                                  int M, int H, const float* hs, float* z) {
    constexpr int P = Row<T>::kPerVec;
    constexpr int kStep = kWave * P;
    const int wave = threadIdx.x / kWave, lane = lane_id();
    int tok[kCorrRows];
    float acc[kCorrRows];
#pragma unroll
    for (int jj = 0; jj < kCorrRows; ++jj) {
        const int j = wave * kCorrRows + jj;
        tok[jj] = j < M ? idx[j] : -1;
        acc[jj] = 0.f;
    }
    for (int k0 = 0; k0 < H; k0 += 2 * kStep) {
        const int ka = k0 + lane * P, kb = ka + kStep;
        const bool oka = ka < H, okb = kb < H;
        u32x4 va[kCorrRows], vb[kCorrRows];
#pragma unroll
        for (int jj = 0; jj < kCorrRows; ++jj) {
            const T* row = C + (size_t)(tok[jj] < 0 ? 0 : tok[jj]) * H;
            const bool on = tok[jj] >= 0;
            va[jj] = (on && oka) ? *reinterpret_cast<const u32x4*>(row + ka) : u32x4{0u, 0u, 0u, 0u};
            vb[jj] = (on && okb) ? *reinterpret_cast<const u32x4*>(row + kb) : u32x4{0u, 0u, 0u, 0u};
        }
        float ha[P], hb[P];
#pragma unroll
        for (int i = 0; i < P; ++i) {
            ha[i] = oka ? hs[ka + i] : 0.f;
            hb[i] = okb ? hs[kb + i] : 0.f;
        }
#pragma unroll
        for (int jj = 0; jj < kCorrRows; ++jj) {
            acc[jj] += Row<T>::dot(va[jj], ha);
            acc[jj] += Row<T>::dot(vb[jj], hb);
        }
    }
#pragma unroll
    for (int jj = 0; jj < kCorrRows; ++jj) {
        const float d = wave_sum(acc[jj]);
        const int j = wave * kCorrRows + jj;
        if (lane == 0 && j < M) z[j] = val[j] + d;
    }
}

// Wave 0: temperature, log-softmax over the M-slice, children sorted by
// (log-prob desc, token asc).  Lane r returns the rank-r child (key 0 when
// r >= M).
__device__ __forceinline__ u64 sorted_children(const float* z, const int32_t* idx, int M, float temp) {
    const int lane = lane_id();
    const bool on = lane < M;
    float zz = on ? z[lane] : -INFINITY;
    if (temp > 0.f) zz = zz / temp;
    const float m = wave_max(zz);
    const float e = on ? expf(zz - m) : 0.f;
    const float ssum = wave_sum(e);
    const float lp = (zz - m) - logf(ssum);
    u64 key = on ? child_key(lp, idx[lane]) : 0ull;
    return wave_sort_desc(key);
}

__device__ __forceinline__ float child_lp_of(u64 k) { return f32_unord((uint32_t)(k >> 32)); }
__device__ __forceinline__ int child_tok_of(u64 k) { return (int)(0xFFFFFFFFu - (uint32_t)k); }

}  // namespace

// Dynamic LDS layout of the node kernel (floats / ints, 16-byte aligned).
NodeLds node_lds_plan(int L, int M, int n, int H) {
    NodeLds p{};
    size_t off = 0;
    auto take = [&](size_t words) {
        size_t at = off;
        off += (words + 3) / 4 * 4;
        return at;
    };
    p.hs = take(H);
    p.zs = take(kMaxM);
    p.sc = take(kMaxN + 1);
    p.par = take(kMaxN + 1);
    p.tidx = take((size_t)L * M);
    p.tval = take((size_t)L * M);
    p.ctok = take((size_t)n * kMaxM);
    p.clp = take((size_t)n * kMaxM);
    p.bytes = off * 4;
    return p;
}

namespace {

// Row sums over the 64 lanes of a wave's 4 per-lane partial dots, reduced
// in transposed form (each exchange halves the values a lane holds): lane l
// ends with the sum of row l / 16, the same in the 16 lanes of a row.
// Lane semantics of the swaps with two operands A, B: permlane32_swap returns
// {[A lower half, B lower half], [A upper half, B upper half]};
// permlane16_swap returns {[A row0, B row0, A row2, B row2],
// [A row1, B row1, A row3, B row3]} (rows of 16 lanes).
__device__ __forceinline__ float wave_rowsum4(const float (&acc)[4]) {
    float s2[2];
#pragma unroll
    for (int i = 0; i < 2; ++i) {  // rows i + 2 * lane bit 5
        const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(acc[i]), __float_as_uint(acc[i + 2]),
                                                        false, false);
        s2[i] = __uint_as_float(r[0]) + __uint_as_float(r[1]);
    }
    // rows bit 4 + 2 * bit 5
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(s2[0]), __float_as_uint(s2[1]), false, false);
    float v = __uint_as_float(r[0]) + __uint_as_float(r[1]);
    v += xor_lane_f<8>(v);
    v += xor_lane_f<4>(v);
    v += xor_lane_f<2>(v);
    v += xor_lane_f<1>(v);
    return v;
}

// Wave 0: z = base logit + correction dot, temperature, log-softmax over the
// M-slice, or over the whole vocabulary when `tz` (the row's tail_lse: the
// uncorrected logits outside the top M, same temperature) is finite; lane j
// holds candidate j's token, base logit and dot and returns its child key
// (log-prob desc, token asc; 0 when j >= M).  Sorted across the wave, lane r
// holds the rank-r child.
__device__ __forceinline__ u64 child_keys_r(float val, float dot, int tok, int M, float temp, float tz) {
    const int lane = lane_id();
    const bool on = lane < M;
    float zz = on ? val + dot : -INFINITY;
    if (temp > 0.f) zz = zz / temp;
    const float m = fmaxf(wave_max(zz), tz);
    const float e = on ? expf(zz - m) : 0.f;
    const float ssum = wave_sum(e) + (tz > -INFINITY ? expf(tz - m) : 0.f);
    const float lp = (zz - m) - logf(ssum);
    return on ? child_key(lp, tok) : 0ull;
}

// What one step hands the next when a workgroup runs all of its request's
// steps (the factorized mode): kept in LDS instead of going through the
// workspace.  The top-M table, child lists, scores and parents stay in the
// node LDS arrays from step to step.
constexpr int kMaxL = 64;  // positions per request (dt_create's limit)
struct StepLds {
    u64 q[kWave];             // queue, one entry per lane
    int32_t rs[kStateWords];  // state record: count, next token, queue size, flags, next depth, parent
    int32_t nidx[kWave];  // the next step's candidate list
    float nval[kWave];
    float tail[kMaxL];    // the rows' tails (full-vocabulary mode)
};

// One expansion step of request blockIdx.x, run by node_threads<MARG>()
// threads.  MARG: factorized (marginal) scoring: the children distribution of
// every node is the log-softmax of the base logits over its M-slice (no GRU
// state, no correction).  PERSIST (with MARG, all steps in one workgroup):
// the state of the previous step comes from `ps` and the LDS arrays instead of
// the workspace (the workspace and outputs are still written).  Waves with no
// further part in the step return early; the step has no workgroup barrier
// after the first such return.
template <typename T, int KS, bool MARG, bool PERSIST = false>
__device__ __forceinline__ void node_step_body(const NodeArgs& a, const NodeLds& lp, int step,
                                               StepLds* ps = nullptr) {
    static_assert(!PERSIST || MARG, "only the factorized mode runs its steps in one workgroup");
    constexpr int NT = node_threads<MARG>();
    constexpr int NW = NT / kWave;
    constexpr int RW = kMaxM / NW;                    // gathered rows per wave
    constexpr int kStageV = kMaxM * kMaxN / (4 * NT);  // 16-byte vectors of table / child list per thread
    extern __shared__ __attribute__((aligned(16))) float lds[];  // (16-byte vector accesses)
    float* hs = lds + lp.hs;
    float* zs = lds + lp.zs;
    float* s_sc = lds + lp.sc;
    int* s_par = (int*)(lds + lp.par);
    int32_t* s_tidx = (int32_t*)(lds + lp.tidx);
    float* s_tval = lds + lp.tval;
    int32_t* s_ctok = (int32_t*)(lds + lp.ctok);
    float* s_clp = lds + lp.clp;
    constexpr int P = Row<T>::kPerVec;       // elements per 16-byte vector
    constexpr int kChunk = 2 * kWave * P;    // K elements of a gathered chunk

    const int b = blockIdx.x;
    const int lane = lane_id();
    const int wave = __builtin_amdgcn_readfirstlane((int)threadIdx.x / kWave);  // wave-uniform
    const int S = a.n + 1;
    const size_t slot0 = (size_t)b * S;
    const int LM = a.L * a.M;
    const int H = a.H;

    // ---- 1. loads.  Round trip 1: the candidate list of the slot expanded
    // now (the previous step left it in nidx/nval; the root takes block
    // position 0 of the table), the gate partial sums, the queue.  Round
    // trip 2, issued as soon as the candidate tokens arrive: the gathered
    // rows of the correction matrix.  Every address is valid whatever the
    // state (tokens clamped to the vocabulary), so no load waits on a test.
    const u64 q_m = PERSIST ? (step == 0 ? 0ull : ps->q[lane]) : a.queue[(size_t)b * kWave + lane];
    // the child keys of slot step - 1, left unsorted by the step that expanded
    // it (sorted below by wave 1; loaded by every wave, from a valid address).
    // The factorized mode, with no gathers to hide a sort behind, sorts a
    // slot's children in the step that expands it, beside the queue update.
    const u64 prev_keys = MARG ? 0ull : a.ckey[(slot0 + (step > 0 ? step - 1 : 0)) * kMaxM + lane];
    // slot `step`'s state: the GRU cell on the K-range partial sums of the
    // preceding contraction, added in K-range order (read at every step; the root
    // takes h0 instead)
    const int k1 = (int)threadIdx.x;  // this thread's state element
    const int kc = k1 < H ? k1 : 0;
    float t[KS][4];
    float bias[6];
    if constexpr (!MARG) {
#pragma unroll
        for (int s2 = 0; s2 < KS; ++s2)
#pragma unroll
            for (int g = 0; g < 4; ++g)
                t[s2][g] = a.partial[((size_t)(s2 * a.B + b) * kGateSlots + g) * H + kc];
#pragma unroll
        for (int g = 0; g < 6; ++g) {
            const void* bp = g < 3 ? a.b_ih : a.b_hh;
            const T* src = bp ? (const T*)bp : (const T*)a.partial;  // any valid address
            const float v = load1<T>(src + (size_t)(g % 3) * H + kc);
            bias[g] = bp ? v : 0.f;
        }
    }
    // (the scheduler keeps the loads above in flight before the candidate
    // list is waited for)
    __builtin_amdgcn_sched_barrier(0);
    // per-request state left by the previous step (one record)
    const i32x4 rs0 = PERSIST ? *reinterpret_cast<const i32x4*>(ps->rs)
                              : *reinterpret_cast<const i32x4*>(a.rstate + (size_t)b * kStateWords);
    const i32x4 rs1 = PERSIST ? *reinterpret_cast<const i32x4*>(ps->rs + 4)
                              : *reinterpret_cast<const i32x4*>(a.rstate + (size_t)b * kStateWords + 4);
    const int rs_depth = rs1[0];
    // full-vocabulary mode: the tails of this request's rows (lane p holds
    // position p's), read from a valid address in either mode
    float tail_l = -INFINITY;
    if (PERSIST) {
        tail_l = a.tail ? ps->tail[min(lane, a.L - 1)] : -INFINITY;
    } else {
        const float* tp = a.tail ? a.tail + (size_t)b * a.L : a.tval;
        const float v = tp[min(lane, a.L - 1)];
        tail_l = a.tail ? v : -INFINITY;
    }
    // folded input projection: the row of this slot's token (r, z, n parts of
    // b_ih + W_ih . x for this thread's state element), from a valid address
    // in either mode
    float xg[3] = {0.f, 0.f, 0.f};
    if constexpr (!MARG) {
        const int xt = min(max(rs0[1], 0), a.V - 1);
        const float* xp = a.table ? a.table + (size_t)xt * 3 * H : a.partial;
#pragma unroll
        for (int g = 0; g < 3; ++g) {
            const float v = xp[(size_t)g * H + kc];
            xg[g] = a.table ? v : 0.f;
        }
    }
    // the parent's state (the GRU's previous state), exact: binary32, or the sum
    // of its three bf16 parts
    const int par = step == 0 ? 0 : min(max(rs1[1], 0), a.n);
    auto parent_state = [&](int kk) {
        if (a.hprev)  // left by the previous step (bf16 path)
            return a.hprev[(size_t)b * H + kk];
        return a.hstate[(slot0 + par) * H + kk];
    };
    const int32_t* ip = step == 0 ? a.tidx + (size_t)b * LM : a.nidx + (size_t)b * kWave;
    const float* vp = step == 0 ? a.tval + (size_t)b * LM : a.nval + (size_t)b * kWave;
    const int jl = min(lane, a.M - 1);
    const bool from_ps = PERSIST && step > 0;
    const int my_tok = min(max(from_ps ? ps->nidx[jl] : ip[jl], 0), a.V - 1);  // candidate `lane` (all waves)
    const float my_val = from_ps ? ps->nval[jl] : vp[jl];
    // the parent's state is loaded before the gathers: loads complete in
    // order, and the GRU cell must not wait for the gathers
    float hp = 0.f;
    if constexpr (!MARG) hp = parent_state(kc);
    // the root's state h0 (first pass), loaded at every step from a valid
    // address: a load inside a branch would make the code after the branch
    // wait for every outstanding load, the gathers included
    float h0v = 0.f;
    if constexpr (!MARG) {
        const float* h0p = a.h0 ? a.h0 + (size_t)b * H : a.partial;
        const float v = h0p[kc];
        h0v = a.h0 ? v : 0.f;
    }
    __builtin_amdgcn_sched_barrier(0);
    // round trip 2: chunk k0 of this wave's RW rows, two vectors per lane and
    // row (positions past H are clamped; their state elements are zero)
    u32x4 cv[RW][2];
    auto gather = [&](int k0) {
        const int ka = min(k0 + lane * P, H - P), kb = min(k0 + (kWave + lane) * P, H - P);
#pragma unroll
        for (int jj = 0; jj < RW; ++jj) {
            const int tk = __builtin_amdgcn_readlane(my_tok, wave * RW + jj);
            const T* row = (const T*)a.C + (size_t)tk * H;
            cv[jj][0] = *reinterpret_cast<const u32x4*>(row + ka);
            cv[jj][1] = *reinterpret_cast<const u32x4*>(row + kb);
        }
    };
    if constexpr (!MARG) gather(0);
    // top-M table of this request, children of slots 0 .. step-1, tree so far
    // (into registers now as 16-byte vectors, into LDS after the state is
    // computed; a table whose rows are not a multiple of 4 entries long is
    // staged element by element below)
    const bool tvec = (LM & 3) == 0;
    i32x4 r_ti[kStageV], r_ct[kStageV];
    f32x4 r_tv[kStageV], r_cl[kStageV];
    const int32_t* ti = a.tidx + (size_t)b * LM;
    const float* tv = a.tval + (size_t)b * LM;
    const int32_t* kt = a.child_tok + slot0 * kMaxM;
    const float* kl = a.child_lp + slot0 * kMaxM;
    const int nkid = step * kMaxM;
#pragma unroll
    for (int u = 0; u < kStageV; ++u) {
        const int e = ((int)threadIdx.x + u * NT) * 4;
        // (with PERSIST the table is staged at step 0 only and the child lists
        // never: the steps write them into LDS themselves)
        const bool te = tvec && e < LM && (!PERSIST || step == 0), ke = !PERSIST && e < nkid;
        r_ti[u] = te ? *reinterpret_cast<const i32x4*>(ti + e) : i32x4{0, 0, 0, 0};
        r_tv[u] = te ? *reinterpret_cast<const f32x4*>(tv + e) : f32x4{0.f, 0.f, 0.f, 0.f};
        r_ct[u] = ke ? *reinterpret_cast<const i32x4*>(kt + e) : i32x4{0, 0, 0, 0};
        r_cl[u] = ke ? *reinterpret_cast<const f32x4*>(kl + e) : f32x4{0.f, 0.f, 0.f, 0.f};
    }
    float r_sc = 0.f;
    int r_par = -1;
    if (!PERSIST && (int)threadIdx.x <= step && threadIdx.x > 0) {
        r_sc = a.scores[slot0 + threadIdx.x];
        r_par = a.parents[slot0 + threadIdx.x];
    }
    const int cnt = step == 0 ? 0 : rs0[0];
    const int gtok = step == 0 ? 0 : rs0[1];
    int qs = step == 0 ? 0 : rs0[2];
    uint32_t flag = step == 0 ? 0u : (uint32_t)rs0[3];
    const int depth = step == 0 ? 0 : rs_depth;
    u64 q = step == 0 ? 0ull : q_m;
    const bool expand = step == 0 || (cnt == step && gtok >= 0);

    // ---- 2. the state of slot `step`, one element per thread and pass (the
    // first pass's operands are already in flight)
    for (int kb0 = 0; kb0 < (MARG ? 0 : H); kb0 += NT) {
        const int kk = kb0 + k1;
        if (kb0 > 0 && kk < H) {  // states wider than NT
#pragma unroll
            for (int s2 = 0; s2 < KS; ++s2)
#pragma unroll
                for (int g = 0; g < 4; ++g)
                    t[s2][g] = a.partial[((size_t)(s2 * a.B + b) * kGateSlots + g) * H + kk];
            hp = parent_state(kk);
#pragma unroll
            for (int g = 0; g < 6; ++g) {
                const void* bp = g < 3 ? a.b_ih : a.b_hh;
                if (bp) bias[g] = load1<T>((const T*)bp + (size_t)(g % 3) * H + kk);
            }
            if (a.table) {
                const int xt = min(max(rs0[1], 0), a.V - 1);
#pragma unroll
                for (int g = 0; g < 3; ++g) xg[g] = a.table[((size_t)xt * 3 + g) * H + kk];
            }
        }
        if (kk >= H) break;
        float hv = 0.f;
        if (step == 0) {
            if (kb0 == 0) hv = h0v;
            else if (a.h0) hv = a.h0[(size_t)b * H + kk];  // states wider than NT
        } else {
            float sum[4];
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                sum[g] = t[0][g];
#pragma unroll
                for (int s2 = 1; s2 < KS; ++s2) sum[g] += t[s2][g];
            }
            if (a.table) {  // the x parts of r, z and the candidate (slot 2 holds none)
                sum[0] += xg[0];
                sum[1] += xg[1];
                sum[2] += xg[2];
            }
            hv = gru_cell_b(sum[0], sum[1], sum[2], sum[3], bias[0], bias[1], bias[2], bias[3], bias[4],
                            bias[5], hp);
        }
        hs[kk] = hv;
        if (expand) {
            if (a.hstate)  // binary32 state (read by the binary32 contraction)
                a.hstate[(slot0 + step) * H + kk] = hv;
            if (a.hsplit) {  // its exact bf16 parts (read by the bf16 contraction)
                uint32_t parts[3];
                split3_bf16(hv, parts);
                uint16_t* pdst = a.hsplit + (slot0 + step) * 3 * (size_t)H + kk;
#pragma unroll
                for (int qq = 0; qq < 3; ++qq) pdst[(size_t)qq * H] = (uint16_t)parts[qq];
            }
        }
    }
#pragma unroll
    for (int u = 0; u < kStageV; ++u) {
        const int e = ((int)threadIdx.x + u * NT) * 4;
        if (tvec && e < LM && (!PERSIST || step == 0)) {
            *reinterpret_cast<i32x4*>(s_tidx + e) = r_ti[u];
            *reinterpret_cast<f32x4*>(s_tval + e) = r_tv[u];
        }
        if (!PERSIST && e < nkid) {
            *reinterpret_cast<i32x4*>(s_ctok + e) = r_ct[u];
            *reinterpret_cast<f32x4*>(s_clp + e) = r_cl[u];
        }
    }
    if (!tvec && (!PERSIST || step == 0)) {
        for (int e = threadIdx.x; e < LM; e += NT) {
            s_tidx[e] = ti[e];
            s_tval[e] = tv[e];
        }
    }
    if (PERSIST ? threadIdx.x == 0 && step == 0 : (int)threadIdx.x <= step) {
        s_sc[threadIdx.x] = threadIdx.x == 0 ? 0.f : r_sc;
        s_par[threadIdx.x] = threadIdx.x == 0 ? -1 : r_par;
    }
    if (!(PERSIST && step > 0)) __syncthreads();  // (later persistent steps stage nothing)

    // Slot step - 1's children sorted by (log-prob desc, token asc), for the
    // sibling pushes from this step on (no earlier step needs them): wave 1
    // sorts them while the gathers are in flight, into the workspace and into
    // the LDS row that the staging above filled with stale data.
    if (!MARG && wave == 1 && step > 0) {
        const u64 kids = wave_sort_desc(prev_keys);
        const int r = step - 1;
        if (lane < a.M) {
            a.child_tok[(slot0 + r) * kMaxM + lane] = child_tok_of(kids);
            a.child_lp[(slot0 + r) * kMaxM + lane] = child_lp_of(kids);
            s_ctok[r * kMaxM + lane] = child_tok_of(kids);
            s_clp[r * kMaxM + lane] = child_lp_of(kids);
        }
    }

    // ---- 3. correction dots of slot `step`'s children (block position = its
    // depth): this wave's RW rows, then a transposed reduction across lanes
    if constexpr (!MARG) {
        if (expand) {
            float acc[RW];
#pragma unroll
            for (int jj = 0; jj < RW; ++jj) acc[jj] = 0.f;
            for (int k0 = 0; k0 < H; k0 += kChunk) {
                if (k0 > 0) gather(k0);  // states wider than one chunk
                const int ka = k0 + lane * P, kb = k0 + (kWave + lane) * P;
                float ha[P], hb[P];  // zero past H (those lanes read a clamped row segment)
#pragma unroll
                for (int i2 = 0; i2 < P; ++i2) {
                    ha[i2] = ka < H ? hs[ka + i2] : 0.f;
                    hb[i2] = kb < H ? hs[kb + i2] : 0.f;
                }
#pragma unroll
                for (int jj = 0; jj < RW; ++jj) {
                    acc[jj] += Row<T>::dot(cv[jj][0], ha);
                    acc[jj] += Row<T>::dot(cv[jj][1], hb);
                }
            }
            static_assert(RW == 4, "the row reduction takes 4 rows per wave");
            const float d = wave_rowsum4(acc);
            if ((lane & 15) == 0) zs[wave * RW + (lane >> 4)] = d;
        }
    }
    if constexpr (!MARG) __syncthreads();  // (the factorized mode has no dots to share)
    // ---- 3. queue.  Wave 0 first takes the pop decision, which needs only the
    // best child of slot `step` (the largest child key; the children are
    // sorted by the next step, or by wave 1 after the decision in the
    // factorized mode), then hands the popped node to the packing waves,
    // which pack the next contraction's activations while wave 0 updates the
    // queue.
    __shared__ int s_dec[2];  // next GRU token (-1 = idle row), parent slot of the popped node
    __shared__ u64 s_keys[kWave];  // (factorized mode) child keys of slot `step`, unsorted
    const float score_step = s_sc[step];
    u64 ckey = 0ull, best = 0ull, top = 0ull;
    int new_cnt = cnt;
    int v_par = -1, pd = 0, pr = 0, ptok = -1;
    int next_depth = 0, next_tok = -1;
    float psc = 0.f;
    const bool pop = wave == 0 && cnt == step && (qs > 0 || expand);
    if (wave == 0) {
        if (expand) {
            const float tz = __int_as_float(
                __builtin_amdgcn_readlane(__float_as_int(tail_l), min(depth, a.L - 1)));
            ckey = child_keys_r(my_val, MARG ? 0.f : zs[lane], my_tok, a.M, a.temp, tz);
            if (MARG) s_keys[lane] = ckey;  // sorted by wave 1 after the decision
            else if (step + 1 < a.n) a.ckey[(slot0 + step) * kMaxM + lane] = ckey;  // sorted by the next step
            best = wave_max_u64(ckey);  // the rank-0 child
            const u64 key = queue_key(score_step + child_lp_of(best), depth + 1, step, 0);
            if (lane == qs) q = key;
            ++qs;
        }
        if (pop) {
            top = wave_max_u64(q);
            pd = qk_depth(top);
            v_par = qk_parent(top);
            pr = qk_rank(top);
            psc = qk_score(top);
            // a child of slot `step` in the queue is its rank-0 child, pushed just now
            ptok = v_par == step ? child_tok_of(best) : s_ctok[v_par * kMaxM + pr];
            const int v = step + 1;
            new_cnt = v;
            next_depth = pd;
            next_tok = pd < a.L && v < a.n ? ptok : -1;
        }
        if (lane == 0) {
            s_dec[0] = next_tok;
            s_dec[1] = v_par;
        }
    }
    __syncthreads();

    if (wave == 1) {
        if (MARG && expand) {  // slot `step`'s children, sorted for the later steps
            const u64 kids = wave_sort_desc(s_keys[lane]);
            const size_t crow = (slot0 + step) * kMaxM;
            if (lane < a.M) {
                a.child_tok[crow + lane] = child_tok_of(kids);
                a.child_lp[crow + lane] = child_lp_of(kids);
                if (PERSIST) {  // row `step` of the LDS child lists (wave 0 reads rows < step)
                    s_ctok[step * kMaxM + lane] = child_tok_of(kids);
                    s_clp[step * kMaxM + lane] = child_lp_of(kids);
                }
            }
        }
        return;  // (otherwise its sort came before the dots)
    }
    if (wave != 0) {
        // ---- 4. row b's activations of the next contraction, packed for its
        // MFMA operands, 8 elements per lane: the popped node's token
        // embedding (waves kXw0 ..) and its parent's state in three exact bf16
        // parts plus binary32 (waves kHw0 ..); zeros for an idle row.  The
        // parent is slot `step` (state in LDS) or an older slot (parts in
        // hsplit).
        constexpr int kXw0 = 2, kXwN = (NW - kXw0 + 1) / 2, kHw0 = kXw0 + kXwN, kHwN = NW - kHw0;
        if (a.hpack && step + 1 < a.n) {
            const int ntok = s_dec[0], vpar = s_dec[1];
            const bool grow = ntok >= 0;
            if (wave < kHw0) {
                if (!a.xpack) return;  // folded input projection: no x part to pack
                const int nv = a.E >> 3;
                for (int i = (wave - kXw0) * kWave + lane; i < nv; i += kXwN * kWave) {
                    u32x4 v = {0u, 0u, 0u, 0u};
                    if (grow) v = *reinterpret_cast<const u32x4*>((const bf16_t*)a.emb + (size_t)ntok * a.E + i * 8);
                    *reinterpret_cast<u32x4*>(a.xpack + pack_index_x(b, i * 8, a.E)) = v;
                }
            } else {
                const int nv = H >> 3;
                for (int i = (wave - kHw0) * kWave + lane; i < nv; i += kHwN * kWave) {
                    const int k = i * 8;
                    uint32_t w[3][4] = {};  // 8 elements of each part, two per word
                    float hv[8];
                    if (grow && vpar == step) {
#pragma unroll
                        for (int e = 0; e < 8; ++e) {
                            hv[e] = hs[k + e];
                            uint32_t p3[3];
                            split3_bf16(hv[e], p3);
#pragma unroll
                            for (int qq = 0; qq < 3; ++qq) w[qq][e >> 1] |= p3[qq] << (16 * (e & 1));
                        }
                    } else if (grow) {
                        const uint16_t* src = a.hsplit + ((slot0 + vpar) * 3) * (size_t)H + k;
#pragma unroll
                        for (int qq = 0; qq < 3; ++qq) {
                            const u32x4 t4 = *reinterpret_cast<const u32x4*>(src + (size_t)qq * H);
                            w[qq][0] = t4.x; w[qq][1] = t4.y; w[qq][2] = t4.z; w[qq][3] = t4.w;
                        }
#pragma unroll
                        for (int e = 0; e < 8; ++e) {  // the exact binary32 state
                            const int sh = 16 * (e & 1);
                            const float p0 = __uint_as_float(((w[0][e >> 1] >> sh) & 0xFFFFu) << 16);
                            const float p1 = __uint_as_float(((w[1][e >> 1] >> sh) & 0xFFFFu) << 16);
                            const float p2 = __uint_as_float(((w[2][e >> 1] >> sh) & 0xFFFFu) << 16);
                            hv[e] = (p0 + p1) + p2;
                        }
                    } else {
#pragma unroll
                        for (int e = 0; e < 8; ++e) hv[e] = 0.f;
                    }
#pragma unroll
                    for (int qq = 0; qq < 3; ++qq)
                        *reinterpret_cast<u32x4*>(a.hpack + pack_index_h(b, qq, k, H)) =
                            u32x4{w[qq][0], w[qq][1], w[qq][2], w[qq][3]};
                    float* hdst = a.hprev + (size_t)b * H + k;
                    *reinterpret_cast<f32x4*>(hdst) = f32x4{hv[0], hv[1], hv[2], hv[3]};
                    *reinterpret_cast<f32x4*>(hdst + 4) = f32x4{hv[4], hv[5], hv[6], hv[7]};
                }
            }
        }
        return;
    }

    // wave 0: the rank-1 child of slot `step` (the sibling pushed when its
    // rank-0 child is popped): the largest key below the rank-0 child's
    const u64 second = expand ? wave_max_u64(ckey == best ? 0ull : ckey) : 0ull;
    if (step == 0) {
        for (int i = lane; i < S; i += kWave) {
            if (i == 0) {
                a.tokens[slot0] = -1;
                a.parents[slot0] = -1;
                a.depths[slot0] = 0;
                a.scores[slot0] = 0.f;
            } else if (i >= 2) {  // slot 1 is written by this step's pop
                a.tokens[slot0 + i] = -1;
                a.parents[slot0 + i] = -1;
                a.depths[slot0 + i] = -1;
                a.scores[slot0 + i] = -INFINITY;
            }
        }
    }
    if (pop) {
        // remove the popped entry, push its next-ranked sibling
        const int holder = (int)__builtin_ctzll(__ballot(q == top));
        const u64 last = bcast_u64(q, qs - 1);
        if (lane == holder) q = last;
        if (lane == qs - 1) q = 0ull;
        --qs;
        const bool has_sib = pr + 1 < a.M;
        // a child of slot `step` popped now is its rank-0 child (pr == 0)
        const float sib_lp = v_par == step ? child_lp_of(second)
                                           : s_clp[v_par * kMaxM + min(pr + 1, kMaxM - 1)];
        if (has_sib) {
            const u64 key = queue_key(s_sc[v_par] + sib_lp, pd, v_par, pr + 1);
            if (lane == qs) q = key;
            ++qs;
        }
        // near tie: the popped score vs every candidate left (binary32 gaps;
        // an exact tie is broken by the queue order and not flagged)
        {
            const float gap = psc - qk_score(q);
            if (__ballot(lane < qs && gap > 0.f && gap < a.eps)) flag |= 1u;
        }
        const int v = step + 1;
        if (lane == 0) {
            a.tokens[slot0 + v] = ptok;
            a.parents[slot0 + v] = v_par;
            a.depths[slot0 + v] = pd;
            a.scores[slot0 + v] = psc;
            a.gru_tok[b] = next_tok;
            a.gru_par[b] = v_par;
            if (PERSIST) {  // slot v's score and parent for the later steps
                s_sc[v] = psc;
                s_par[v] = v_par;
            }
        }
        if (next_tok >= 0) {  // the next step expands v: hand over its candidates
            const int jm = min(lane, a.M - 1);
            a.nidx[(size_t)b * kWave + lane] = s_tidx[pd * a.M + jm];
            a.nval[(size_t)b * kWave + lane] = s_tval[pd * a.M + jm];
            if (PERSIST) {
                ps->nidx[lane] = s_tidx[pd * a.M + jm];
                ps->nval[lane] = s_tval[pd * a.M + jm];
            }
        }
    } else if (lane == 0) {
        a.gru_tok[b] = -1;
        a.gru_par[b] = 0;
    }
    a.queue[(size_t)b * kWave + lane] = q;
    if (lane == 0) {
        int32_t* rs = a.rstate + (size_t)b * kStateWords;
        *reinterpret_cast<i32x4*>(rs) = i32x4{new_cnt, next_tok, qs, (int)flag};
        *reinterpret_cast<i32x4*>(rs + 4) = i32x4{next_depth, v_par < 0 ? 0 : v_par, 0, 0};
        a.count[b] = new_cnt;
        a.flags[b] = flag;
    }
    if (PERSIST) {  // read by every wave at the start of the next step
        ps->q[lane] = q;
        if (lane == 0) {
            *reinterpret_cast<i32x4*>(ps->rs) = i32x4{new_cnt, next_tok, qs, (int)flag};
            *reinterpret_cast<i32x4*>(ps->rs + 4) = i32x4{next_depth, v_par < 0 ? 0 : v_par, 0, 0};
        }
    }

    // ---- 5. ancestor-only mask after the last step
    if (step == a.n - 1) {
        if (lane == 0 && new_cnt == step + 1) s_par[step + 1] = v_par;
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "workgroup");
        for (int i = lane; i < S; i += kWave) {
            uint8_t* row = a.mask + ((size_t)b * S + i) * S;
            u64 bits_lo = 0ull;  // slots 0..63
            bool bit64 = false;  // slot 64 (only when n = 64)
            if (i <= new_cnt) {
                for (int j = i; j >= 0; j = j == 0 ? -1 : s_par[j]) {
                    if (j < 64) bits_lo |= 1ull << j;
                    else bit64 = true;
                }
            }
            for (int j = 0; j < S; ++j)
                row[j] = (uint8_t)(j < 64 ? ((bits_lo >> j) & 1ull) : (bit64 ? 1 : 0));
        }
    }
}

template <typename T, int KS, bool MARG>
__global__ __launch_bounds__(node_threads<MARG>()) void node_step_kernel(NodeArgs a, NodeLds lp, int step) {
    node_step_body<T, KS, MARG>(a, lp, step);
}

// The factorized mode's whole expansion in one launch: without the batched
// contraction nothing ties the requests together between steps, so each
// workgroup runs its request's n steps back to back, handing the queue, state
// record and candidate list from step to step in LDS (and keeping the table,
// child lists, scores and parents there), a workgroup barrier between steps.
template <typename T>
__global__ __launch_bounds__(node_threads<true>()) void marginal_build_kernel(NodeArgs a, NodeLds lp) {
    __shared__ StepLds ps;
    if (a.tail && (int)threadIdx.x < a.L) ps.tail[threadIdx.x] = a.tail[(size_t)blockIdx.x * a.L + threadIdx.x];
    __syncthreads();
    for (int step = 0; step < a.n; ++step) {
        node_step_body<T, 1, true, true>(a, lp, step, &ps);
        __syncthreads();
    }
}

template <typename T>
__global__ __launch_bounds__(kCorrThreads) void correct_kernel(const int32_t* tidx, const float* tval,
                                                               const T* C, const float* h,
                                                               const int32_t* pos, int32_t* tok_out,
                                                               float* lp_out, int L, int H, int M,
                                                               float temp) {
    __shared__ float hs[kMaxH];
    __shared__ float zs[kMaxM];
    __shared__ int32_t si[kMaxM];
    __shared__ float sv[kMaxM];
    const int b = blockIdx.x;
    for (int k = threadIdx.x; k < H; k += kCorrThreads) hs[k] = h[(size_t)b * H + k];
    const size_t trow = ((size_t)b * L + pos[b]) * M;
    if (threadIdx.x < M) {
        si[threadIdx.x] = tidx[trow + threadIdx.x];
        sv[threadIdx.x] = tval[trow + threadIdx.x];
    }
    __syncthreads();
    correction_logits<T>(C, si, sv, M, H, hs, zs);
    __syncthreads();
    if (threadIdx.x >= kWave) return;
    const u64 kids = sorted_children(zs, si, M, temp);
    const int lane = lane_id();
    if (lane < M) {
        tok_out[(size_t)b * M + lane] = child_tok_of(kids);
        lp_out[(size_t)b * M + lane] = child_lp_of(kids);
    }
}

// ============================================================================
// Fused pipelined expansion (bf16).  One launch per expansion step; its grid
// holds `ng` contraction workgroups (blocks 0 .. ng-1) and one node workgroup
// per request (blocks ng .. ng+B-1), all of 512 threads, on separate CUs.
//
// The GRU update of node v needs gi(v) = W_ih . Emb[tok(v)] (its token's input
// projection) and gh(p) = W_hh . h(p) (its parent's recurrent projection).
// Launch t's contraction computes, per request, gi of one token (x row) and
// gh of the node that request expanded at launch t - 1 (h row, kept per slot
// in the workspace).  Its node workgroup meanwhile expands the node popped at
// t - 1 with what earlier launches contracted, so the contraction is off the
// expansion's dependency chain.  The x row of launch t + 1 is chosen by the
// node workgroup of launch t: after its pop, the queue's best candidate is
// the next pop unless the node expanded at t + 1 has a better child, so that
// candidate's token is contracted ahead (a prediction); when a pop takes the
// newest child instead, the popped node's own token is contracted at t + 1
// and the request waits one launch (it expands at t + 2).  Every launch after
// the first expands at most one node per request, so a call runs n + 2
// launches; a request that has used its one spare launch and is not ready
// waits inside the launch for that launch's contraction (a counter the
// contraction workgroups raise; bounded spin) instead of idling.  Results are
// the stepped path's, up to binary32 rounding order of the gate sums.
// ============================================================================

constexpr int kPipeThreads = 512;
constexpr int kMaxB = 64;      // requests of a fused call
constexpr int kPipeMaxKs = 3;  // partial sums per kind (x part, h part) of a gate sum
constexpr int kPipeWaves = kPipeThreads / kWave;    // 8
constexpr int kPipeRows = kMaxM / kPipeWaves;       // 8 gathered rows per wave
constexpr unsigned kPipeSpinLimit = 1u << 18;       // bounded wait for a launch's contraction (~0.3 s)
constexpr uint32_t kPipeTimeoutFlag = 0x80000000u;  // flags bit: such a wait timed out
// dynamic LDS a fused launch may take: a CU's 160 KB less the static
// variables of the node role (and headroom)
constexpr size_t kPipeMaxDynLds = 160 * 1024 - 256;

// Buffer p[i] of a launch-parity pair, by selection: indexing the kernel
// argument's array with a run-time index would copy the argument to scratch.
template <typename P>
__device__ __forceinline__ P by_parity(P const (&p)[2], int i) {
    return i ? p[1] : p[0];
}

// Agent-scope loads (coherent across XCDs) of the gate sums that a waiting
// node workgroup reads in the launch that computes them.
__device__ __forceinline__ float ld_agent(const float* p) {
    return __uint_as_float(__hip_atomic_load((unsigned*)p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
}
__device__ __forceinline__ float2 ld_agent2(const float* p) {  // (8-byte aligned)
    const unsigned long long v =
        __hip_atomic_load((unsigned long long*)p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    return make_float2(__uint_as_float((uint32_t)v), __uint_as_float((uint32_t)(v >> 32)));
}
__device__ __forceinline__ int ld_agent_i(const int32_t* p) {
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_agent_i(int32_t* p, int v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// ---- hand-over inside one launch (the persistent launch, and a request that
// waits for its launch's contraction).  Each XCD has its own L2, written back
// to memory only at the end of a kernel (and invalidated at the start of
// one).  Data that another XCD reads in the same launch is therefore stored
// with the device-scope cache policy (sc1: written through to the
// device-coherent level), and once the stores are complete (vmcnt(0)) the
// workgroup's own flag word is set to the step it finished.  The reader uses
// sc1 loads where its XCD may hold an older copy of the line (the gate sums,
// rewritten every other step); data written once per launch and read only
// after its flag (a slot's state) is read through the caches, provided that
// nothing reads it before it is written.  No L2 writeback or invalidation is
// needed, what a workgroup keeps for itself stays cached, and no two
// workgroups update one word (same-address atomics from every workgroup
// serialize).
constexpr int kCpolSc1 = 16;  // cache-policy operand of buffer and LDS-copy builtins: sc1
// Buffer resource over a buffer whose offsets fit 32 bits (uniform base)
__device__ __forceinline__ __amdgpu_buffer_rsrc_t coherent_rsrc(const void* base) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, 0x7fffffff, 0x00020000);
}
__device__ __forceinline__ void st_through(__amdgpu_buffer_rsrc_t r, size_t byte_off, u32x4 v) {
    __builtin_amdgcn_raw_buffer_store_b128(v, r, (int)byte_off, 0, kCpolSc1);
}
__device__ __forceinline__ void st_through2(__amdgpu_buffer_rsrc_t r, size_t byte_off, float x, float y) {
    typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
    __builtin_amdgcn_raw_buffer_store_b64(u32x2{__float_as_uint(x), __float_as_uint(y)}, r, (int)byte_off, 0,
                                          kCpolSc1);
}
// Wait (wave 0, bounded) until every flag f[0 .. n) (n <= 256) is at least
// target -- lane l reads flags l, l + 64, ... with device-coherent loads --
// then the workgroup barrier.  A wait that runs out, or finds that another
// wait ran out, raises *perr and returns: every workgroup still runs to its
// end.
// poll_flags: the same wait by one wave, without the barrier.
// The flags' first loads, issued ahead of a wait (lane l: flags l, l + 64,
// ..., the last flag again past n; no branch, so that a later wait counts
// exactly the loads issued after these).
struct FlagPeek {
    unsigned v[4];
};
__device__ __forceinline__ FlagPeek peek_flags(const unsigned* f, int n) {
    const int l = lane_id();
    FlagPeek p;
#pragma unroll
    for (int i = 0; i < 4; ++i)
        p.v[i] = __hip_atomic_load(f + min(l + i * kWave, n - 1), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    return p;
}
__device__ __forceinline__ void poll_flags(const unsigned* f, int n, unsigned target, unsigned* perr,
                                           FlagPeek p = FlagPeek{{0u, 0u, 0u, 0u}}) {
    unsigned spins = 0;
    for (;;) {
        bool ok = true;
#pragma unroll
        for (int i = 0; i < 4; ++i) ok &= p.v[i] >= target;
        if (__ballot(!ok) == 0ull) break;
        if ((++spins & 63u) == 0u &&
            (spins >= kPipeSpinLimit || __hip_atomic_load(perr, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT))) {
            if (lane_id() == 0) __hip_atomic_fetch_or(perr, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            break;
        }
        __builtin_amdgcn_s_sleep(1);
        p = peek_flags(f, n);  // (the loads issued together)
    }
}
__device__ __forceinline__ void wait_flags(const unsigned* f, int n, unsigned target, unsigned* perr) {
    if (threadIdx.x < kWave) poll_flags(f, n, target, perr, peek_flags(f, n));
    __syncthreads();
}
__device__ __forceinline__ void set_flag(unsigned* f, unsigned v) {
    __hip_atomic_store(f, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// A node workgroup's x flag for the contraction of step s (one word per
// request and step parity): s (bits 19 ..), whether the request waits in
// step s (bit 18) and the token of step s's x row + 1 (bits 0 .. 17; 0:
// none).  The word of step s is >= xflag_word(s, -1, false); the word of step
// s - 2 in the same slot is below it.
constexpr int kXflagStep = 19;
constexpr int kPersMaxV = (1 << 18) - 1;  // tokens the x flag can carry
__host__ __device__ constexpr unsigned xflag_word(int step, int tok, bool wait) {
    return ((unsigned)step << kXflagStep) | ((wait ? 1u : 0u) << 18) | (unsigned)(tok + 1);
}
// Wait (wave 0, bounded) for the B x flags of step s, then put the x rows'
// offsets in the embedding table (token * E; token 0 where none, and past B)
// into s_roff[0 .. 64) unless it is NULL, and whether any request waits into
// *s_any; then the workgroup barrier.
__device__ __forceinline__ void wait_xflags(const unsigned* f, int B, int V, int E, int s, unsigned* perr,
                                            int32_t* s_roff, int* s_any) {
    if (threadIdx.x < kWave) {
        const int l = (int)threadIdx.x;
        const unsigned target = xflag_word(s, -1, false);
        unsigned v = target, spins = 0;
        for (;;) {
            v = l < B ? __hip_atomic_load(f + l, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) : target;
            if (__ballot(v < target) == 0ull) break;
            if ((++spins & 63u) == 0u &&
                (spins >= kPipeSpinLimit || __hip_atomic_load(perr, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT))) {
                if (l == 0) __hip_atomic_fetch_or(perr, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                break;
            }
            __builtin_amdgcn_s_sleep(1);
        }
        const int tok1 = (int)(v & ((1u << 18) - 1u));
        if (s_roff) s_roff[l] = (l < B && tok1 > 0 ? min(tok1 - 1, V - 1) : 0) * E;  // (no x row: token 0)
        const bool any = __ballot(l < B && ((v >> 18) & 1u)) != 0ull;
        if (l == 0) *s_any = any;
    }
    __syncthreads();
}
// A node workgroup's h flag for the contraction of step s (one word per
// request and step parity): s (bits 8 ..) and the slot whose state is the h
// row of step s, + 1 (bits 0 .. 7; 0: none).
__host__ __device__ constexpr unsigned hflag_word(int step, int slot) {
    return ((unsigned)step << 8) | (unsigned)(slot + 1);
}
// Wait (wave 0, bounded) for the B h flags of step s, then put each row's
// slot into s_slot[0 .. 64) (-1 where none, and past B) and the offset of its
// state among the per-slot states [B][S][H] into s_roff (row 0's first slot
// where none); then the workgroup barrier.
__device__ __forceinline__ void wait_hflags(const unsigned* f, int B, int S, int H, int s, unsigned* perr,
                                            int32_t* s_roff, int32_t* s_slot) {
    if (threadIdx.x < kWave) {
        const int l = (int)threadIdx.x;
        const unsigned target = hflag_word(s, -1);
        unsigned v = target, spins = 0;
        for (;;) {
            v = l < B ? __hip_atomic_load(f + l, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) : target;
            if (__ballot(v < target) == 0ull) break;
            if ((++spins & 63u) == 0u &&
                (spins >= kPipeSpinLimit || __hip_atomic_load(perr, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT))) {
                if (l == 0) __hip_atomic_fetch_or(perr, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                break;
            }
            __builtin_amdgcn_s_sleep(1);
        }
        const int sl = l < B ? (int)(v & 255u) - 1 : -1;
        const bool ok = sl >= 0 && sl < S;
        s_slot[l] = ok ? sl : -1;
        s_roff[l] = ok ? (l * S + sl) * H : 0;
    }
    __syncthreads();
}

// The four quarters of each unit tile (waves 4 u + 0 .. 3) added in order,
// quarter 0 first, and stored (when `store`): every wave leaves its sums in
// LDS ([wave][rb * 3 + slot][lane]); wave 4 u + q then adds up and stores the
// slot vectors j = q, q + 4, ... of the unit tile.  Lane l holds units 4 (l /
// 16) .. + 3 of row l % 16 of each row block.  gi by launch parity, gh by the
// slot of the state (hsl_r: thread i < B holds row i's slot, loaded before
// the tile and put into LDS here, after it).  COH: the stores are written
// through (read by other workgroups in the same launch).
template <int RB, bool COH>
__device__ __forceinline__ void gate_sums(const PipeArgs& a, int t, int ug, int kind, int ksub, int hsl_r, bool store,
                                          gate::f32x4 (&acc)[RB][3], float* lds, int* s_hsl) {
    __syncthreads();  // every wave is done with the staged activations
    const int wave = __builtin_amdgcn_readfirstlane((int)threadIdx.x / kWave), lane = lane_id();
    const int u = wave / gate::kT32Quarters, qt = wave % gate::kT32Quarters;
    gate::f32x4* red = reinterpret_cast<gate::f32x4*>(lds);
#pragma unroll
    for (int rb = 0; rb < RB; ++rb)
#pragma unroll
        for (int sl = 0; sl < 3; ++sl) red[(wave * RB * 3 + rb * 3 + sl) * kWave + lane] = acc[rb][sl];
    if ((int)threadIdx.x < a.B) s_hsl[threadIdx.x] = hsl_r;
    __syncthreads();
    if (!store) return;
    // (the fields are read into values first: selecting between fields of
    // the kernel argument would copy the argument to scratch)
    float* const gi = a.gi;
    float* const gh = a.gh;
    const int B = a.B, H = a.H, ksx = a.ksx, ksh = a.ksh, S = a.n + 1, par = t & 1;
    const int unit = ug * 32 + u * 16 + (lane >> 4) * 4;
    const __amdgpu_buffer_rsrc_t rs = coherent_rsrc(kind == 0 ? (const void*)gi : (const void*)gh);
#pragma unroll
    for (int j0 = 0; j0 < RB * 3; j0 += gate::kT32Quarters) {
        const int j = j0 + qt;  // (wave-uniform)
        if (j >= RB * 3) break;
        const int rb = j / 3, sl = j % 3;
        gate::f32x4 sum = red[((u * gate::kT32Quarters) * RB * 3 + j) * kWave + lane];
#pragma unroll
        for (int q = 1; q < gate::kT32Quarters; ++q)
            sum += red[((u * gate::kT32Quarters + q) * RB * 3 + j) * kWave + lane];
        const int row = rb * 16 + (lane & 15);
        const int hsl = kind ? s_hsl[min(row, B - 1)] : 0;
        if (row >= B || (kind && (hsl < 0 || hsl >= S))) continue;
        const size_t off = kind == 0 ? (((size_t)(par * ksx + ksub) * B + row) * 3 + sl) * H + unit
                                     : ((((size_t)row * S + hsl) * ksh + ksub) * 3 + sl) * H + unit;
        if constexpr (COH) st_through(rs, off * 4, __builtin_bit_cast(u32x4, sum));
        else *reinterpret_cast<gate::f32x4*>((kind == 0 ? gi : gh) + off) = sum;
    }
}

// A node workgroup's record between the steps of the persistent launch, in
// LDS after the slots' expansion steps: queue, unsorted child keys, handed-over
// candidates, state words, the two x-row tokens; then the gate biases b_ih,
// b_hh as binary32 [6][H] (staged at step 0).
struct PersLds {
    u64* q;
    u64* ckey;
    int32_t* nidx;
    float* nval;
    int32_t* rs;
    int32_t* xt;
    float* bias;
};
__host__ __device__ constexpr size_t pers_lds_bytes(int H) {
    return 64 * 8 * 2 + 64 * 4 * 2 + kStateWords * 4 + 16 + (size_t)6 * H * 4;
}
__host__ __device__ inline size_t pers_lds_offset(const NodeLds& lp, int n) {
    return lp.bytes + (((size_t)n + 1) * 4 + 15) / 16 * 16;  // (bytes; after s_exp)
}
__device__ __forceinline__ PersLds pers_lds(float* lds, const NodeLds& lp, int n) {
    char* p = reinterpret_cast<char*>(lds) + pers_lds_offset(lp, n);
    PersLds r;
    r.q = reinterpret_cast<u64*>(p);
    r.ckey = r.q + 64;
    r.nidx = reinterpret_cast<int32_t*>(r.ckey + 64);
    r.nval = reinterpret_cast<float*>(r.nidx + 64);
    r.rs = reinterpret_cast<int32_t*>(r.nval + 64);
    r.xt = r.rs + kStateWords;
    r.bias = reinterpret_cast<float*>(r.xt + 4);
    return r;
}

// Contraction role: 32 hidden units x one K range of launch t's rows (the
// 32-unit tile of gate_tile.h: the activations staged in LDS once per
// workgroup).  Its x waves' sums are the x part of gates (r, z, n), its h
// waves' sums the h part; the two halves of each are added in LDS (first
// half first) and stored: gi by launch parity, gh by the slot of the state.
template <int WM, int RB>
__device__ __forceinline__ void pipe_gate(const PipeArgs& a, int t, float* lds) {
    const int groups = a.H / 32;
    const int ug = (int)blockIdx.x % groups, kw = (int)blockIdx.x / groups;
    const int kind = kw >= a.ksx, ksub = kind ? kw - a.ksx : kw, nsub = kind ? a.ksh : a.ksx;
    if (t == 0) {
        // no rows yet: clear this call's per-launch counters and flags, and
        // lay this workgroup's weights out in operand tiles for the later
        // launches (beside the root expansions)
        if (blockIdx.x == 0)
            for (int i = threadIdx.x; i < a.T; i += kPipeThreads) {
                a.done[i] = 0u;
                a.active[i] = 0;
                a.active[a.T + i] = 0;
            }
        GruGatesArgs g{};
        g.W_ih = a.W_ih;
        g.W_hh = a.W_hh;
        g.E = a.E;
        g.H = a.H;
        g.wpack = a.wpack;
        gate::t32_pack_weights(g, ug, kind, ksub, nsub);
        return;
    }
    // after the last launch nothing expands: its sums are read only by requests
    // waiting in it (published then).  (The flag is read in this branch only,
    // by a load of its own: a plain load would be shared with the one below
    // and waited for here, at the start of every launch.)
    if (t == a.T - 1 &&
        __hip_atomic_load(a.active + a.T + t, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == 0)
        return;
    const int par = t & 1;
    // this launch's flags: some row needs the contraction (launch 1 always
    // has rows); some request waits for its sums in this launch, so they are
    // published (release) and the workgroup counted -- otherwise they are
    // read from launch t + 1 on, after the launch boundary, and plain stores
    // suffice.  Their loads overlap the contraction, which runs either way
    // (its inputs are always in bounds; without rows nothing is stored).
    const int act = a.active[t], publish = a.active[a.T + t];
    // each row's state slot: loaded now, stored into LDS after the tile
    // (a store would wait for the load here)
    __shared__ int s_hsl[kMaxB];
    const int hsl_r = (int)threadIdx.x < a.B ? by_parity(a.hslot, par)[threadIdx.x] : -1;
    GruGatesArgs g{};
    g.xpack = by_parity(a.xpack, par);
    g.hpack = by_parity(a.hpack, par);
    g.W_ih = a.W_ih;
    g.W_hh = a.W_hh;
    g.B = a.B;
    g.E = a.E;
    g.H = a.H;
    g.ksplit = 1;  // (unused by this tile)
    g.dtype = 1;
    g.wpack = a.wpack;
    g.wmode = WM;
    gate::f32x4 acc[RB][3];
    gate::tile32_lds<WM, RB>(g, ug, kind, ksub, nsub, reinterpret_cast<gate::u32x4*>(lds), acc);
    gate_sums<RB, false>(a, t, ug, kind, ksub, hsl_r, t == 1 || act != 0, acc, lds, s_hsl);
    if (publish) {
        // every store of the workgroup has reached the L2; thread 0 writes the
        // L2 back (agent-scope release) and counts the workgroup
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        __syncthreads();
        if (threadIdx.x == 0) {
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
            __hip_atomic_fetch_add(a.done + t, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
    }
}

// Contraction role of the persistent launch: the workgroup's weights are
// loaded into registers once, then every step t = 1 .. T - 1 waits for the
// node workgroups' rows of step t - 1 -- an x workgroup for their x tokens
// (it reads the embedding rows itself), an h workgroup for the slots of their
// states (it reads the binary32 states and splits them itself) --, contracts
// and raises its flag.  The last step runs only if some request waits in it.
// Both read their rows through the caches: the embedding table is never
// written, and a slot's state is written once per launch (written through,
// before the flag that names it) and read only after.
template <int KIND, int RB>
__device__ __forceinline__ void pers_gate_loop(const PipeArgs& a, GruGatesArgs& g, const gate::T32Wave& r, int ug,
                                               int ksub, float* lds) {
    __shared__ int s_hsl[kMaxB];
    __shared__ int32_t s_roff[kWave];  // the rows' offsets (row blocks of 16)
    __shared__ int32_t s_slot[kWave];  // h rows: the slot of each row's state
    __shared__ int s_any;              // some request waits in this step
    gate::bf16x8 w[gate::t32_xbatch(RB)][3];
    gate::t32_load_weights<KIND, false, RB>(g, r, w);
    for (int t = 1; t < a.T; ++t) {
        const int par = t & 1;
        // (the wait bits of the last step travel with the x tokens)
        if (KIND == 0 || t == a.T - 1)
            wait_xflags(a.xflag + par * a.B, a.B, a.V, a.E, t, a.perr, KIND == 0 ? s_roff : nullptr, &s_any);
        if (KIND == 1) wait_hflags(a.hflag + par * a.B, a.B, a.n + 1, a.H, t, a.perr, s_roff, s_slot);
        if (t == a.T - 1 && !s_any) break;
        const int hsl_r = KIND == 1 && (int)threadIdx.x < a.B ? s_slot[threadIdx.x] : -1;
        gate::f32x4 acc[RB][3];
        gate::t32_contract<KIND, false, RB, 0, true>(g, r, reinterpret_cast<gate::u32x4*>(lds), w, acc, s_roff,
                                                     a.hstate);
        gate_sums<RB, true>(a, t, ug, KIND, ksub, hsl_r, true, acc, lds, s_hsl);
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // the sums are written through
        __syncthreads();
        if (threadIdx.x == 0) set_flag(a.gflag + blockIdx.x, (unsigned)t);
    }
}
template <int RB>
__device__ __forceinline__ void pers_gate(const PipeArgs& a, float* lds) {
    const int groups = a.H / 32;
    const int ug = (int)blockIdx.x % groups, kw = (int)blockIdx.x / groups;
    const int kind = kw >= a.ksx, ksub = kind ? kw - a.ksx : kw, nsub = kind ? a.ksh : a.ksx;
    GruGatesArgs g{};
    g.x = a.emb;
    g.W_ih = a.W_ih;
    g.W_hh = a.W_hh;
    g.B = a.B;
    g.E = a.E;
    g.H = a.H;
    g.ksplit = 1;
    g.dtype = 1;
    const gate::T32Wave r = gate::t32_wave(g, ug, kind, ksub, nsub);
    if (kind == 0) pers_gate_loop<0, RB>(a, g, r, ug, ksub, lds);
    else pers_gate_loop<1, RB>(a, g, r, ug, ksub, lds);
}

// The state hs ([H] binary32 in LDS) in three exact bf16 parts, as request
// b's h row of the contraction of launch parity pn (pack_index_h): wave w of
// four takes the 8-element vectors w * 64 + lane, + 256, ...
__device__ __forceinline__ void pack_state(const PipeArgs& a, const float* hs, int b, int pn, int w, int lane) {
    const int H = a.H, nv = H >> 3;
    uint16_t* const hq = by_parity(a.hpack, pn);
    for (int i = w * kWave + lane; i < nv; i += 4 * kWave) {
        const int k = i * 8;
        uint32_t v[3][4] = {};
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            uint32_t p3[3];
            split3_bf16(hs[k + e], p3);
#pragma unroll
            for (int qq = 0; qq < 3; ++qq) v[qq][e >> 1] |= p3[qq] << (16 * (e & 1));
        }
#pragma unroll
        for (int qq = 0; qq < 3; ++qq) {
            const u32x4 x = u32x4{v[qq][0], v[qq][1], v[qq][2], v[qq][3]};
            *reinterpret_cast<u32x4*>(hq + pack_index_h(b, qq, k, H)) = x;
        }
    }
}

// Node role: request b's step at launch t.  PERS: step t of the persistent
// launch -- it first waits for the contraction of step t - 1 and reads the
// gate sums, writes the new state through and names its slot in the h flag,
// and the next x row's token in the x flag (its own records stay in LDS and
// its XCD's caches).
enum PipeMode { kRoot, kExpand, kWait, kTrivial, kIdle, kDone };

template <bool PERS>
__device__ __forceinline__ void pipe_node(const PipeArgs& a, const NodeLds& lp, int t, float* lds, int tid) {
    constexpr int NT = kPipeThreads, RW = kPipeRows;
    constexpr int P = 8;                    // bf16 elements per 16-byte vector

    constexpr int kStageV = kMaxM * kMaxN / (4 * NT);  // 16-byte vectors of table / child list per thread
    float* hs = lds + lp.hs;
    float* zs = lds + lp.zs;
    float* s_sc = lds + lp.sc;
    int* s_par = (int*)(lds + lp.par);
    int32_t* s_tidx = (int32_t*)(lds + lp.tidx);
    float* s_tval = lds + lp.tval;
    int32_t* s_ctok = (int32_t*)(lds + lp.ctok);
    float* s_clp = lds + lp.clp;
    int32_t* s_exp = (int32_t*)(lds + lp.bytes / 4);  // [n+1] launch that expanded each slot
    __shared__ int s_dec[4];  // x-row token and h-row slot of the next launch, mode
    // persistent launch: the request's record from step to step, in LDS (the
    // top-M table, child lists, scores, parents and expansion steps stay in
    // their LDS arrays)
    PersLds ps = pers_lds(lds, lp, a.n);

    const int b = (int)blockIdx.x - a.ng;
    const int lane = tid & (kWave - 1);
    const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
    // persistent launch: the first loads of the wait for the contraction of
    // step t - 1, issued before the step's own (their round trip overlaps them)
    FlagPeek peek{{0u, 0u, 0u, 0u}};
    if (PERS && t >= 2 && wave == 0) peek = peek_flags(a.gflag, a.ng);
    const int S = a.n + 1, H = a.H, M = a.M, LM = a.L * a.M;
    const size_t slot0 = (size_t)b * S;
    const int pt = t & 1, pn = (t + 1) & 1;  // this launch's parity; the next's (= the previous one's)
    const int KSX = a.ksx, KSH = a.ksh;  // partial sums of the x part and of the h part
    // (two adjacent gate sums; the persistent launch's are written through by
    // another XCD)
    auto ld_sum2 = [](const float* p) { return PERS ? ld_agent2(p) : *reinterpret_cast<const float2*>(p); };
    // ---- round trip 1 (every address valid in every mode); the persistent
    // launch takes the request's record from LDS
    i32x4 rs0, rs1;
    u64 q_m;
    int xt_prev, xt_cur;  // launch t-1's x row, this launch's
    const int jl = min(lane, M - 1);
    int my_tok;
    float my_val;
    if constexpr (PERS) {
        rs0 = *reinterpret_cast<const i32x4*>(ps.rs);
        rs1 = *reinterpret_cast<const i32x4*>(ps.rs + 4);
        q_m = ps.q[lane];
        xt_prev = ps.xt[pn];
        xt_cur = ps.xt[pt];
        my_tok = min(max(ps.nidx[jl], 0), a.V - 1);  // (step 0: the root's, put there before the steps)
        my_val = ps.nval[jl];
    } else {
        rs0 = *reinterpret_cast<const i32x4*>(a.rstate + (size_t)b * kStateWords);
        rs1 = *reinterpret_cast<const i32x4*>(a.rstate + (size_t)b * kStateWords + 4);
        q_m = a.queue[(size_t)b * kWave + lane];
        xt_prev = by_parity(a.xtok, pn)[b];
        xt_cur = by_parity(a.xtok, pt)[b];
        const int32_t* ip = t == 0 ? a.tidx + (size_t)b * LM : a.nidx + (size_t)b * kWave;
        const float* vp = t == 0 ? a.tval + (size_t)b * LM : a.nval + (size_t)b * kWave;
        my_tok = min(max(ip[jl], 0), a.V - 1);
        my_val = vp[jl];
    }
    // this thread's state elements k1 = 2 tid and k2 = k1 + 1 (H even, H <= 2 NT)
    const int k1 = 2 * tid, k2 = k1 + 1;
    const int kc1 = k1 < H ? k1 : 0;  // (pair loads: elements kc1, kc1 + 1)
    float gi[2][kPipeMaxKs][3];
    auto load_gi = [&]() {
#pragma unroll
        for (int s2 = 0; s2 < kPipeMaxKs; ++s2)
#pragma unroll
            for (int g = 0; g < 3; ++g) {
                const size_t base = (((size_t)(pn * KSX + min(s2, KSX - 1)) * a.B + b) * 3 + g) * H;
                const float2 v = ld_sum2(a.gi + base + kc1);
                gi[0][s2][g] = v.x;
                gi[1][s2][g] = v.y;
            }
    };
    if constexpr (!PERS) load_gi();
    // (loads without branches, from a stand-in address when a pointer is
    // NULL, so that every path issues the same loads: the in-order load
    // counters then let round trip 2 wait for exactly what it needs)
    // (the persistent launch keeps the biases in LDS and reads h0 in the cell)
    float bias[2][6];
#pragma unroll
    for (int g = 0; g < 6; ++g) {
        if constexpr (PERS) break;
        const void* bp = g < 3 ? a.b_ih : a.b_hh;
        // stand-in: W_ih, [3H, E] with E >= 1, holds at least 3H elements
        const bf16_t* src = bp ? (const bf16_t*)bp : (const bf16_t*)a.W_ih;
        const uint32_t two = *reinterpret_cast<const uint32_t*>(src + (size_t)(g % 3) * H + kc1);
        bias[0][g] = bp ? __uint_as_float(two << 16) : 0.f;
        bias[1][g] = bp ? __uint_as_float(two & 0xFFFF0000u) : 0.f;
    }
    float h0v[2] = {0.f, 0.f};
    if (!PERS) {
        // stand-in: W_ih, [3H, E] bf16 with E >= 1, holds 2H floats (not the
        // per-slot states: the persistent launch's contraction reads those
        // through the caches, and nothing may cache a state before it is
        // written)
        const float* h0p = a.h0 ? a.h0 + (size_t)b * H : (const float*)a.W_ih;
        const float2 v = *reinterpret_cast<const float2*>(h0p + kc1);
        h0v[0] = a.h0 ? v.x : 0.f;
        h0v[1] = a.h0 ? v.y : 0.f;
    }
    float tail_l = -INFINITY;
    {
        const float* tp = a.tail ? a.tail + (size_t)b * a.L : a.tval;
        const float v = tp[min(lane, a.L - 1)];
        tail_l = a.tail ? v : -INFINITY;
    }
    // top-M table, sorted child lists, scores, parents and expansion launches
    // of every slot (rows of slots not yet filled are never read)
    const bool tvec = (LM & 3) == 0;
    i32x4 r_ti[kStageV], r_ct[kStageV];
    f32x4 r_tv[kStageV], r_cl[kStageV];
    const int32_t* ti = a.tidx + (size_t)b * LM;
    const float* tv = a.tval + (size_t)b * LM;
    const int32_t* kt = a.child_tok + slot0 * kMaxM;
    const float* kl = a.child_lp + slot0 * kMaxM;
    const int nkid = a.n * kMaxM;
#pragma unroll
    for (int u = 0; u < kStageV; ++u) {
        const int e = (tid + u * NT) * 4;
        // (the persistent launch copies the table at step 0 without these)
        const bool te = !PERS && tvec && e < LM, ke = !PERS && t > 0 && e < nkid;
        r_ti[u] = te ? *reinterpret_cast<const i32x4*>(ti + e) : i32x4{0, 0, 0, 0};
        r_tv[u] = te ? *reinterpret_cast<const f32x4*>(tv + e) : f32x4{0.f, 0.f, 0.f, 0.f};
        r_ct[u] = ke ? *reinterpret_cast<const i32x4*>(kt + e) : i32x4{0, 0, 0, 0};
        r_cl[u] = ke ? *reinterpret_cast<const f32x4*>(kl + e) : f32x4{0.f, 0.f, 0.f, 0.f};
    }
    float r_sc = 0.f;
    int r_par = -1, r_exp = 0;
    if (!PERS && t > 0 && tid < S) {
        r_sc = a.scores[slot0 + tid];
        r_par = a.parents[slot0 + tid];
        r_exp = a.exp_at[slot0 + tid];
    }
    __builtin_amdgcn_sched_barrier(0);

    // ---- the request's state and this launch's mode (uniform)
    const int cnt = t == 0 ? 0 : rs0[0];
    const int cur = t == 0 ? 0 : (rs0[1] < 0 ? -1 : min(rs0[1], a.n));
    int qs = t == 0 ? 0 : rs0[2];
    uint32_t flag = t == 0 ? 0u : (uint32_t)rs0[3];
    const int unsorted = t == 0 || rs1[0] < 0 || rs1[0] >= a.n ? -1 : rs1[0];
    const int ctok = t == 0 ? -1 : rs1[1];
    const int cpar = t == 0 ? -1 : min(max(rs1[2], 0), a.n);
    const int cdepth = t == 0 ? 0 : (rs1[3] & 0xffff);
    // launch that expanded cur's parent (recorded at cur's pop)
    const int pexp = t == 0 ? 0 : (int)((unsigned)rs1[3] >> 16);
    u64 q = t == 0 ? 0ull : q_m;
    // a node to expand (its GRU inputs may not be ready yet): its correction
    // rows are gathered at once, whatever the readiness turns out to be
    const bool cand = t > 0 && cnt < a.n && cur >= 0 && cdepth < a.L;

    // ---- round trip 2: the gathered correction rows (first: the critical
    // path runs through them), the parent's gh and state, the unsorted keys
    u32x4 cv[RW][2];
    auto gather = [&](int k0) {
        const int ka = min(k0 + lane * P, H - P), kb = min(k0 + (kWave + lane) * P, H - P);
#pragma unroll
        for (int jj = 0; jj < RW; ++jj) {
            const int tk = __builtin_amdgcn_readlane(my_tok, wave * RW + jj);
            const bf16_t* row = (const bf16_t*)a.C + (size_t)tk * H;
            cv[jj][0] = *reinterpret_cast<const u32x4*>(row + ka);
            cv[jj][1] = *reinterpret_cast<const u32x4*>(row + kb);
        }
    };
    const int cp = t == 0 ? 0 : cpar;
    float gh[2][kPipeMaxKs][3];
    float hp[2];
    const float* ghp = a.gh + (slot0 + cp) * (size_t)KSH * 3 * H;
    auto load_gh = [&]() {
#pragma unroll
        for (int s2 = 0; s2 < kPipeMaxKs; ++s2)
#pragma unroll
            for (int g = 0; g < 3; ++g) {
                const size_t o = ((size_t)min(s2, KSH - 1) * 3 + g) * H;
                const float2 v = ld_sum2(ghp + o + kc1);
                gh[0][s2][g] = v.x;
                gh[1][s2][g] = v.y;
            }
    };
    if constexpr (!PERS) load_gh();
    {
        const float2 v = *reinterpret_cast<const float2*>(a.hstate + (slot0 + cp) * H + kc1);
        hp[0] = v.x;
        hp[1] = v.y;
    }
    const u64 prev_keys = PERS ? ps.ckey[lane] : a.ckey[(slot0 + (unsorted >= 0 ? unsorted : 0)) * kMaxM + lane];
    if (t == 0 || cand) gather(0);
    if constexpr (PERS) {
        // with the gathers in flight: wait for the contraction of step t - 1
        // (its sums, and the end of its reads of the activation buffers that
        // this step rewrites; step 1 reads no sums and writes buffers no
        // contraction has read), then read its sums.  Meanwhile wave 1 sorts
        // the children of the slot grown at step t - 1, for the sibling
        // pushes of this and later steps.
        if (t >= 2 || unsorted >= 0) {
            if (t >= 2 && wave == 0) poll_flags(a.gflag, a.ng, (unsigned)(t - 1), a.perr, peek);
            if (wave == 1 && unsorted >= 0) {
                const u64 kids = wave_sort_desc(prev_keys);
                if (lane < M) {
                    s_ctok[unsorted * kMaxM + lane] = child_tok_of(kids);
                    s_clp[unsorted * kMaxM + lane] = child_lp_of(kids);
                }
            }
            __syncthreads();
        }
        load_gi();
        load_gh();
    }
    // this launch's mode (uniform over the workgroup)
    int mode;
    if (t == 0) mode = kRoot;
    else if (cnt >= a.n || cur < 0) mode = kDone;
    else if (cdepth >= a.L) mode = kTrivial;
    else if (xt_prev == ctok && pexp <= t - 2) mode = kExpand;  // gi and the parent's gh are ready
    else if (a.n - cnt <= a.T - 1 - t) mode = kIdle;            // a spare launch is left: expand at t + 1
    else mode = kWait;                                           // none left: take this launch's
    const bool grow = mode == kRoot || mode == kExpand || mode == kWait;
    const int ecur = mode == kRoot ? 0 : cur;  // the slot expanded (or popped trivially) now

    // ---- stage into LDS (the persistent launch: once, at step 0)
    // (the persistent launch stages the table before its first step)
    const bool stage = !PERS;
#pragma unroll
    for (int u = 0; u < kStageV; ++u) {
        const int e = (tid + u * NT) * 4;
        if (!PERS && tvec && e < LM) {
            *reinterpret_cast<i32x4*>(s_tidx + e) = r_ti[u];
            *reinterpret_cast<f32x4*>(s_tval + e) = r_tv[u];
        }
        if (!PERS && e < nkid) {
            *reinterpret_cast<i32x4*>(s_ctok + e) = r_ct[u];
            *reinterpret_cast<f32x4*>(s_clp + e) = r_cl[u];
        }
    }
    if (stage && !tvec)
        for (int e = tid; e < LM; e += NT) {
            s_tidx[e] = ti[e];
            s_tval[e] = tv[e];
        }
    if (stage && tid < S) {
        s_sc[tid] = tid == 0 ? 0.f : r_sc;
        s_par[tid] = tid == 0 ? -1 : r_par;
        s_exp[tid] = r_exp;
    }

    // ---- wait for this launch's contraction (bounded), then take its sums
    if (mode == kWait) {
        if constexpr (PERS) {  // every contraction workgroup finished step t
            wait_flags(a.gflag, a.ng, (unsigned)t, a.perr);
        } else {
            if (tid == 0) {
                unsigned spins = 0;
                while (__hip_atomic_load(a.done + t, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) < (unsigned)a.ng &&
                       ++spins < kPipeSpinLimit)
                    __builtin_amdgcn_s_sleep(2);
                s_dec[3] = spins >= kPipeSpinLimit;
                __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");  // (lines of the sums cached earlier are stale)
            }
            __syncthreads();
            if (s_dec[3]) flag |= kPipeTimeoutFlag;
        }
#pragma unroll
        for (int s2 = 0; s2 < kPipeMaxKs; ++s2)
#pragma unroll
            for (int g = 0; g < 3; ++g) {
                const size_t base = (((size_t)(pt * KSX + min(s2, KSX - 1)) * a.B + b) * 3 + g) * H;
                const float2 v = ld_agent2(a.gi + base + kc1);
                gi[0][s2][g] = v.x;
                gi[1][s2][g] = v.y;
                const size_t o = ((size_t)min(s2, KSH - 1) * 3 + g) * H;
                const float2 w2 = ld_agent2(ghp + o + kc1);
                gh[0][s2][g] = w2.x;
                gh[1][s2][g] = w2.y;
            }
        // complete the reloads here (vmcnt(0) alone): after this branch the
        // cell then waits only for the loads it uses on either path, not for
        // the gathered rows issued after them on the other path
        __builtin_amdgcn_s_waitcnt(0x0F70);
    }

    // ---- the expanded node's state: GRU cell (the root takes h0)
    float hv2[2] = {0.f, 0.f};
    if (grow) {
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            const int kk = u == 0 ? k1 : k2;
            if (kk >= H) continue;
            float hv = h0v[u];
            if (PERS && mode == kRoot) hv = a.h0 ? a.h0[(size_t)b * H + kk] : 0.f;
            if (PERS && mode != kRoot) {
#pragma unroll
                for (int g = 0; g < 6; ++g) bias[u][g] = ps.bias[g * H + kk];
            }
            if (mode != kRoot) {
                float sr = 0.f, sz = 0.f, snx = 0.f, snh = 0.f;
#pragma unroll
                for (int s2 = 0; s2 < kPipeMaxKs; ++s2)
                    if (s2 < KSX) {
                        sr += gi[u][s2][0];
                        sz += gi[u][s2][1];
                        snx += gi[u][s2][2];
                    }
                float hr = 0.f, hz = 0.f;
#pragma unroll
                for (int s2 = 0; s2 < kPipeMaxKs; ++s2)
                    if (s2 < KSH) {
                        hr += gh[u][s2][0];
                        hz += gh[u][s2][1];
                        snh += gh[u][s2][2];
                    }
                hv = gru_cell_b(sr + hr, sz + hz, snx, snh, bias[u][0], bias[u][1], bias[u][2], bias[u][3],
                                bias[u][4], bias[u][5], hp[u]);
            }
            hs[kk] = hv;
            if constexpr (PERS) hv2[u] = hv;
            else a.hstate[(slot0 + (mode == kRoot ? 0 : cur)) * H + kk] = hv;
        }
        // (the persistent launch: written through, read by the contraction
        // of step t + 1 once the h flag names the slot)
        if (PERS && k1 < H) st_through2(coherent_rsrc(a.hstate), ((slot0 + ecur) * H + k1) * 4, hv2[0], hv2[1]);
    }
    __syncthreads();

    // the previously expanded slot's children, sorted for the sibling pushes
    // of this and later launches (wave 1, while the gathers are in flight;
    // the persistent launch sorts them during its wait for the contraction)
    if (!PERS && wave == 1 && unsorted >= 0) {
        const u64 kids = wave_sort_desc(prev_keys);
        if (lane < M) {
            a.child_tok[(slot0 + unsorted) * kMaxM + lane] = child_tok_of(kids);
            a.child_lp[(slot0 + unsorted) * kMaxM + lane] = child_lp_of(kids);
            s_ctok[unsorted * kMaxM + lane] = child_tok_of(kids);
            s_clp[unsorted * kMaxM + lane] = child_lp_of(kids);
        }
    }

    // the queue's two best entries before this launch's pushes (wave 0, while
    // the gathers are in flight): a pop takes the first or the expanded
    // node's best child, and the next best is among the two, that child and
    // the popped entry's sibling
    u64 qa = 0ull, qb = 0ull;
    if (wave == 0) {
        qa = wave_max_u64(q);
        qb = wave_max_u64(q == qa ? 0ull : q);
    }

    // ---- correction dots of the expanded node's children
    if (grow) {
        float acc[RW];
#pragma unroll
        for (int jj = 0; jj < RW; ++jj) acc[jj] = 0.f;
        {  // one chunk: the fused plan has H <= kChunk
            const int ka = lane * P, kb = (kWave + lane) * P;
            // (H is a multiple of 32: a lane's 8 elements are all in range or
            // all past H, where its gathered vector repeats another's)
            float ha[P], hb[P];
            const f32x4 a0 = *reinterpret_cast<const f32x4*>(hs + min(ka, H - P));
            const f32x4 a1 = *reinterpret_cast<const f32x4*>(hs + min(ka, H - P) + 4);
            const f32x4 b0 = *reinterpret_cast<const f32x4*>(hs + min(kb, H - P));
            const f32x4 b1 = *reinterpret_cast<const f32x4*>(hs + min(kb, H - P) + 4);
            const bool ia = ka < H, ib = kb < H;
#pragma unroll
            for (int i2 = 0; i2 < 4; ++i2) {
                ha[i2] = ia ? a0[i2] : 0.f;
                ha[4 + i2] = ia ? a1[i2] : 0.f;
                hb[i2] = ib ? b0[i2] : 0.f;
                hb[4 + i2] = ib ? b1[i2] : 0.f;
            }
#pragma unroll
            for (int jj = 0; jj < RW; ++jj) {
                acc[jj] += Row<bf16_t>::dot(cv[jj][0], ha);
                acc[jj] += Row<bf16_t>::dot(cv[jj][1], hb);
            }
        }
        const float lo[4] = {acc[0], acc[1], acc[2], acc[3]};
        const float hi[4] = {acc[4], acc[5], acc[6], acc[7]};
        const float d0 = wave_rowsum4(lo), d1 = wave_rowsum4(hi);
        if ((lane & 15) == 0) {
            zs[wave * RW + (lane >> 4)] = d0;
            zs[wave * RW + 4 + (lane >> 4)] = d1;
        }
    }
    // (persistent launch: every wave's stores of the state are complete
    // before its h flag goes out)
    if constexpr (PERS) asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();

    // ---- queue (wave 0): push the expanded node's best child, pop the next
    // node, choose the next launch's contraction rows.  The pop is the larger
    // of qa and that child (keys are unique); what a pop of qa reads is
    // fetched before the children are known, and the queue is left as a push
    // and a swap-remove of the popped entry would leave it.
    u64 ckey = 0ull, best = 0ull, second = 0ull;
    int new_cnt = cnt, new_cur = cur, v_par = -1, pd = 0, pr = 0, ptok = -1;
    float psc = 0.f;
    int xtok_next = -1, hslot_next = grow ? ecur : -1;
    bool wait_next = false;  // launch t + 1 will find the popped node not ready and no launch to spare
    int vexp_rec = 0;        // launch that expanded the popped node's parent
    const bool pops = mode == kRoot || mode == kExpand || mode == kWait || mode == kTrivial;
    if (PERS && wave == 4 && lane == 0) {
        // persistent launch: the next step's h row is this state (its slot
        // in the flag word; the state contraction of step t + 1 starts on it,
        // not on the end of the step)
        set_flag(a.hflag + pn * a.B + b, hflag_word(t + 1, grow ? ecur : -1));
    }
    if (wave == 0) {
        const int edepth = mode == kRoot ? 0 : cdepth;
        // qa and qb: parent, rank, depth; their tokens, qa's sibling and the
        // rows a pop of qa hands over (LDS reads issued ahead; an empty entry
        // reads slot n's rows, unused)
        const int pa = min(qk_parent(qa), a.n), ra = qk_rank(qa), da = qk_depth(qa);
        const int pb = min(qk_parent(qb), a.n), rb = qk_rank(qb);
        const int jm = min(lane, M - 1);
        const int tok_qa = s_ctok[pa * kMaxM + min(ra, kMaxM - 1)];
        const int tok_qb = s_ctok[pb * kMaxM + min(rb, kMaxM - 1)];
        const int tok_sb = s_ctok[pa * kMaxM + min(ra + 1, kMaxM - 1)];
        const float lp_sb = s_clp[pa * kMaxM + min(ra + 1, kMaxM - 1)];
        const float sc_pa = s_sc[pa];
        const int exp_pa = s_exp[pa];
        const float sc_e = s_sc[ecur];
        const int rowa = min(edepth + 1, a.L - 1) * M + jm, rowb = min(da, a.L - 1) * M + jm;
        const int hi_a = s_tidx[rowa], hi_b = s_tidx[rowb];
        const float hv_a = s_tval[rowa], hv_b = s_tval[rowb];
        u64 kbest = 0ull;
        if (grow) {
            const float tz = __int_as_float(
                __builtin_amdgcn_readlane(__float_as_int(tail_l), min(edepth, a.L - 1)));
            ckey = child_keys_r(my_val, zs[lane], my_tok, M, a.temp, tz);
            if constexpr (PERS) ps.ckey[lane] = ckey;  // sorted at the next step
            else a.ckey[(slot0 + ecur) * kMaxM + lane] = ckey;  // sorted at the next launch
            best = wave_max_u64(ckey);
            second = wave_max_u64(ckey == best ? 0ull : ckey);
            kbest = queue_key(sc_e + child_lp_of(best), edepth + 1, ecur, 0);
        }
        const int qs0 = qs;  // entries before this launch's pushes
        if (pops && (grow || qs0 > 0)) {
            const bool take_a = grow && kbest > qa;  // the expanded node's best child is popped
            const u64 top = take_a ? kbest : qa;
            pd = qk_depth(top);
            v_par = qk_parent(top);
            pr = qk_rank(top);
            psc = qk_score(top);
            ptok = take_a ? child_tok_of(best) : tok_qa;
            const int v = cnt + 1;
            new_cnt = v;
            new_cur = v;
            // the popped entry's next-ranked sibling, and the best entry left
            const bool sib = pr + 1 < M;
            u64 ksib = 0ull, nb;
            int ntok;
            if (take_a) {  // kbest never enters the queue; its sibling takes lane qs0
                if (sib) ksib = queue_key(sc_e + child_lp_of(second), pd, ecur, 1);
                if (sib && lane == qs0) q = ksib;
                qs = qs0 + (sib ? 1 : 0);
                nb = qa;
                ntok = tok_qa;
                if (ksib > nb) {
                    nb = ksib;
                    ntok = child_tok_of(second);
                }
            } else {  // qa's lane takes the last entry (kbest when pushed)
                const int holder = (int)__builtin_ctzll(__ballot(q == qa));
                const int last = grow ? qs0 : qs0 - 1;
                const u64 klast = grow ? kbest : bcast_u64(q, last);
                if (lane == holder) q = klast;
                if (lane == last) q = 0ull;
                qs = last;
                if (sib) {
                    ksib = queue_key(sc_pa + lp_sb, pd, v_par, pr + 1);
                    if (lane == qs) q = ksib;
                    ++qs;
                }
                nb = qb;
                ntok = tok_qb;
                if (kbest > nb) {
                    nb = kbest;
                    ntok = child_tok_of(best);
                }
                if (ksib > nb) {
                    nb = ksib;
                    ntok = tok_sb;
                }
            }
            {  // near tie: the popped score vs every candidate left
                const float gap = psc - qk_score(q);
                if (__ballot(lane < qs && gap > 0.f && gap < a.eps)) flag |= 1u;
            }
            if (lane == 0) {
                a.tokens[slot0 + v] = ptok;
                a.parents[slot0 + v] = v_par;
                a.depths[slot0 + v] = pd;
                a.scores[slot0 + v] = psc;
                s_sc[v] = psc;
                s_par[v] = v_par;
            }
            if (pd < a.L) {  // hand over the popped node's candidates
                if constexpr (PERS) {
                    ps.nidx[lane] = take_a ? hi_a : hi_b;
                    ps.nval[lane] = take_a ? hv_a : hv_b;
                } else {
                    a.nidx[(size_t)b * kWave + lane] = take_a ? hi_a : hi_b;
                    a.nval[(size_t)b * kWave + lane] = take_a ? hv_a : hv_b;
                }
            }
            // the next launch's x row: the popped node's token when it cannot
            // expand at t + 1, else the token of the best entry left (the
            // likely pop of launch t + 1)
            if (v >= a.n) {
                xtok_next = -1;
            } else {
                const int vexp = take_a ? t : exp_pa;
                vexp_rec = vexp;
                const bool ready_next = pd >= a.L || (t > 0 && ptok == xt_cur && vexp <= t - 1);
                if (ready_next) xtok_next = nb != 0ull ? ntok : -1;
                else xtok_next = ptok;
                // (the mode test of launch t + 1, decided here: not ready, and
                // no idle launch left)
                wait_next = !ready_next && !(a.n - v <= a.T - 2 - t);
            }
        } else if (pops) {  // the candidate tree is exhausted
            new_cur = -1;
        } else if (mode == kIdle) {
            // cur expands at t + 1: contract the likely pop after it
            xtok_next = qa != 0ull ? tok_qa : -1;
        }
        if (lane == 0) {
            s_dec[0] = xtok_next;
            s_dec[1] = hslot_next;
        }
        if constexpr (PERS) {
            // the next step's x row (the contraction reads its embedding row
            // by this token) and whether the request waits in it, in the flag
            // word itself (one store, nothing to complete first)
            if (lane == 0)
                set_flag(a.xflag + pn * a.B + b, xflag_word(t + 1, xtok_next, wait_next && t + 1 < a.T));
        }
    }
    __syncthreads();

    if (wave != 0) {
        if constexpr (!PERS) {
            // ---- the next launch's activations (waves 1 .. 7): the x row
            // (waves 1 .. 3) and the expanded node's state in three exact
            // bf16 parts (waves 4 .. 7)
            const int xn = s_dec[0], hn = s_dec[1];
            if (wave < 4) {
                if (xn < 0) return;
                uint16_t* const xp = by_parity(a.xpack, pn);
                const int nv = a.E >> 3;
                const size_t row = (size_t)min(xn, a.V - 1) * a.E;  // (a token of the request's tables: < V)
                for (int i = (wave - 1) * kWave + lane; i < nv; i += 3 * kWave) {
                    const u32x4 v = *reinterpret_cast<const u32x4*>((const bf16_t*)a.emb + row + i * 8);
                    *reinterpret_cast<u32x4*>(xp + pack_index_x(b, i * 8, a.E)) = v;
                }
            } else if (hn >= 0) {
                pack_state(a, hs, b, pn, wave - 4, lane);
            }
            return;
        }
    } else {
        // ---- wave 0: the request's record for the next launch, outputs
        if (t == 0) {  // the empty tree around the root
            for (int i = lane; i < S; i += kWave) {
                if (i == 0) {
                    a.tokens[slot0] = -1;
                    a.parents[slot0] = -1;
                    a.depths[slot0] = 0;
                    a.scores[slot0] = 0.f;
                } else if (i >= 2 || new_cnt < 1) {  // slot 1 is this launch's pop
                    a.tokens[slot0 + i] = -1;
                    a.parents[slot0 + i] = -1;
                    a.depths[slot0 + i] = -1;
                    a.scores[slot0 + i] = -INFINITY;
                }
            }
            if (lane == 0) {  // (the parity launch 1 reads as "previous")
                if constexpr (PERS) ps.xt[pt] = -1;
                else by_parity(a.xtok, pt)[b] = -1;
            }
        }
        if constexpr (PERS) ps.q[lane] = q;
        else a.queue[(size_t)b * kWave + lane] = q;
        if (lane == 0) {
            if constexpr (PERS) {
                if (grow) s_exp[ecur] = t;
                ps.xt[pn] = xtok_next;
            } else {
                if (grow) a.exp_at[slot0 + ecur] = t;
                by_parity(a.xtok, pn)[b] = xtok_next;
            }
            if constexpr (PERS) {  // (its rows and flags went out after the cell and the queue)
                if (t == a.T - 1 && __hip_atomic_load(a.perr, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT))
                    flag |= kPipeTimeoutFlag;  // some wait of the launch ran out
            } else {
                by_parity(a.hslot, pn)[b] = hslot_next;
                if ((xtok_next >= 0 || hslot_next >= 0) && t + 1 < a.T) a.active[t + 1] = 1;
                if (wait_next && t + 1 < a.T) a.active[a.T + t + 1] = 1;  // its contraction publishes
            }
            const int nd = new_cur == cur && !pops ? (rs1[3] & 0xffff) | (pexp << 16) : pd | (vexp_rec << 16);
            const int ntok = new_cur == cur && !pops ? ctok : ptok;
            const int npar = new_cur == cur && !pops ? cpar : v_par;
            int32_t* rs = PERS ? ps.rs : a.rstate + (size_t)b * kStateWords;
            *reinterpret_cast<i32x4*>(rs) = i32x4{new_cnt, new_cur, qs, (int)flag};
            *reinterpret_cast<i32x4*>(rs + 4) = i32x4{grow ? ecur : -1, ntok, npar < 0 ? 0 : npar, nd};
            a.count[b] = new_cnt;
            a.flags[b] = flag;
        }

        // ---- ancestor-only mask, at the call's last launch
        if (t == a.T - 1) {
            __builtin_amdgcn_wave_barrier();
            __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "workgroup");
            for (int i = lane; i < S; i += kWave) {
                uint8_t* row = a.mask + ((size_t)b * S + i) * S;
                u64 bits_lo = 0ull;
                bool bit64 = false;
                if (i <= new_cnt) {
                    for (int j = i; j >= 0; j = j == 0 ? -1 : s_par[j]) {
                        if (j < 64) bits_lo |= 1ull << j;
                        else bit64 = true;
                    }
                }
                for (int j = 0; j < S; ++j)
                    row[j] = (uint8_t)(j < 64 ? ((bits_lo >> j) & 1ull) : (bit64 ? 1 : 0));
            }
        }
    }
    if constexpr (PERS) __syncthreads();  // (the next step reuses the LDS)
}

template <int WM, int RB>
__global__ __launch_bounds__(kPipeThreads) void pipe_kernel(PipeArgs a, NodeLds lp, int t) {
    extern __shared__ __attribute__((aligned(16))) float lds[];  // (16-byte vector accesses)
    if ((int)blockIdx.x < a.ng) pipe_gate<WM, RB>(a, t, lds);
    else pipe_node<false>(a, lp, t, lds, (int)threadIdx.x);
}

// The persistent launch: the same grid and roles, every step of the call.
// A contraction workgroup keeps its weights in registers; a node workgroup
// keeps its request's records in its XCD's caches.  Step t's contraction
// waits for the node workgroups' step t - 1 and the node workgroups' step t
// for step t - 1's contraction (and a waiting request for step t's), so the
// two roles run one step apart, as the launches do.  Co-residency of the
// grid is guaranteed by the cooperative launch; every wait is bounded.
template <int RB>
__global__ __launch_bounds__(kPipeThreads) void pers_kernel(PipeArgs a, NodeLds lp) {
    extern __shared__ __attribute__((aligned(16))) float lds[];  // (16-byte vector accesses)
    if (a.tclock && threadIdx.x == 0)
        __hip_atomic_fetch_min(a.tclock, wall_clock64(), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if ((int)blockIdx.x < a.ng) {
        pers_gate<RB>(a, lds);
    } else {
        {  // the root's candidates, where every step reads the node's; the
            // request's top-M table and the gate biases (binary32)
            const int b = (int)blockIdx.x - a.ng, LM = a.L * a.M, H = a.H, tid = (int)threadIdx.x;
            const PersLds ps = pers_lds(lds, lp, a.n);
            if (tid < a.M) {
                ps.nidx[tid] = a.tidx[(size_t)b * LM + tid];
                ps.nval[tid] = a.tval[(size_t)b * LM + tid];
            }
            const int32_t* ti = a.tidx + (size_t)b * LM;
            const float* tv = a.tval + (size_t)b * LM;
            int32_t* s_tidx = (int32_t*)(lds + lp.tidx);
            float* s_tval = lds + lp.tval;
            if ((LM & 3) == 0) {
                for (int e = tid * 4; e < LM; e += 4 * kPipeThreads) {
                    *reinterpret_cast<i32x4*>(s_tidx + e) = *reinterpret_cast<const i32x4*>(ti + e);
                    *reinterpret_cast<f32x4*>(s_tval + e) = *reinterpret_cast<const f32x4*>(tv + e);
                }
            } else {
                for (int e = tid; e < LM; e += kPipeThreads) {
                    s_tidx[e] = ti[e];
                    s_tval[e] = tv[e];
                }
            }
            // the slots' scores, parents and expansion steps (slot 0: the root)
            for (int i = tid; i <= a.n; i += kPipeThreads) {
                lds[lp.sc + i] = 0.f;
                reinterpret_cast<int*>(lds + lp.par)[i] = -1;
                reinterpret_cast<int32_t*>(lds + lp.bytes / 4)[i] = 0;
            }
            // (8 bf16 per thread and load; H % 32 == 0)
            for (int e = tid * 8; e < 6 * H; e += 8 * kPipeThreads) {
                const bf16_t* bp = (const bf16_t*)(e < 3 * H ? a.b_ih : a.b_hh);
                const int o = e < 3 * H ? e : e - 3 * H;
                const u32x4 v = bp ? *reinterpret_cast<const u32x4*>(bp + o) : u32x4{0u, 0u, 0u, 0u};
                const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    ps.bias[e + 2 * i] = __uint_as_float(w[i] << 16);
                    ps.bias[e + 2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
                }
            }
            __syncthreads();
        }
        for (int t = 0; t < a.T; ++t) {
            // (the thread index through an opaque copy in each step: what is
            // derived from it, such as the per-lane addresses, is then
            // computed in the step and not held across the steps)
            int tid = (int)threadIdx.x;
            asm volatile("" : "+v"(tid));
            pipe_node<true>(a, lp, t, lds, tid);
        }
    }
    if (a.tclock) {
        __syncthreads();
        if (threadIdx.x == 0)
            __hip_atomic_fetch_max(a.tclock + 1, wall_clock64(), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
}

}  // namespace

template <typename T>
hipError_t launch_node_t(const NodeArgs& a, const NodeLds& lp, int step, hipStream_t stream,
                         LaunchEvents ev) {
    const dim3 grid(a.B), block(node_threads<false>());
    const unsigned shm = (unsigned)lp.bytes;
    if (a.marginal) return hipErrorInvalidValue;  // the factorized mode runs marginal_build_kernel
    switch (a.ksplit) {
#define DT_KS(K) \
    case K: return launch_kernel(node_step_kernel<T, K, false>, grid, block, shm, stream, ev, a, lp, step);
        DT_KS(1) DT_KS(2) DT_KS(3) DT_KS(4) DT_KS(5) DT_KS(6)
#undef DT_KS
        default: return hipErrorInvalidValue;
    }
}

hipError_t launch_node_step(const NodeArgs& a, const NodeLds& lp, int step, hipStream_t stream,
                            LaunchEvents ev) {
    if (a.B == 0) return hipSuccess;
    return a.dtype == 1 ? launch_node_t<bf16_t>(a, lp, step, stream, ev)
                        : launch_node_t<float>(a, lp, step, stream, ev);
}

hipError_t launch_marginal_build(const NodeArgs& a, const NodeLds& lp, hipStream_t stream, LaunchEvents ev) {
    if (a.B == 0) return hipSuccess;
    const dim3 grid(a.B), block(node_threads<true>());
    const unsigned shm = (unsigned)lp.bytes;
    return a.dtype == 1 ? launch_kernel(marginal_build_kernel<bf16_t>, grid, block, shm, stream, ev, a, lp)
                        : launch_kernel(marginal_build_kernel<float>, grid, block, shm, stream, ev, a, lp);
}

hipError_t launch_correct(const int32_t* tidx, const float* tval, const void* C, const float* h,
                          const int32_t* pos, int32_t* tok_sorted, float* lp_sorted, int B, int L,
                          int H, int M, int dtype, float temp, hipStream_t stream) {
    if (B == 0) return hipSuccess;
    if (dtype == 1)
        correct_kernel<bf16_t><<<B, kCorrThreads, 0, stream>>>(tidx, tval, (const bf16_t*)C, h, pos,
                                                               tok_sorted, lp_sorted, L, H, M, temp);
    else
        correct_kernel<float><<<B, kCorrThreads, 0, stream>>>(tidx, tval, (const float*)C, h, pos,
                                                              tok_sorted, lp_sorted, L, H, M, temp);
    return hipGetLastError();
}


PipePlan pipe_plan(int B, int L, int E, int H, int M, int n) {
    PipePlan p{};
    if (B < 1 || B > 64 || H > 2 * kPipeThreads || H % 32 || E % 32) return p;  // ng = 0: not applicable
    // contraction workgroups of 32 units x one share of the x part or of the
    // h part, and the requests' node workgroups, together at most one per CU
    const int groups = H / 32;
    const int per = std::min(2 * kPipeMaxKs, (256 - B) / groups);  // shares per 32 units
    if (per < 2) return p;
    p.ksh = per / 2;
    p.ksx = per - p.ksh;
    p.ng = groups * per;
    p.rb = gate::row_blocks(B);
    if (!gate::t32_fits(E / 32, H / 32, p.ksx, p.ksh, p.rb)) return PipePlan{};  // one weight batch per wave
    const NodeLds lp = node_lds_plan(L, M, n, H);
    const size_t node = pers_lds_offset(lp, n) + pers_lds_bytes(H);  // + the slots' expansion launches, the record
    const size_t red = (size_t)kPipeWaves * p.rb * 3 * kWave * 16;  // the waves' sums
    const size_t gates = std::max(gate::t32_act_bytes(E / 32, H / 32, p.ksx, p.ksh, p.rb), red);
    p.lds = std::max(node, gates);
    if (p.lds > kPipeMaxDynLds) return PipePlan{};  // does not fit one CU's LDS
    return p;
}

hipError_t launch_pipe_step(const PipeArgs& a, const PipePlan& pp, const NodeLds& lp, int t, hipStream_t stream,
                            LaunchEvents ev) {
    if (a.B == 0) return hipSuccess;
    const dim3 grid(pp.ng + a.B), block(kPipeThreads);
    const unsigned shm = (unsigned)pp.lds;
    const int wm = 2;  // (launch 0 lays the weights out in operand tiles; the later ones read them)
#define DT_PIPE(WM, RB)                                                                                    \
    if (wm == WM && pp.rb == RB) {                                                                         \
        static unsigned granted = 0;  /* dynamic LDS bytes allowed so far (grows only) */                \
        if (shm > granted) {                                                                               \
            const hipError_t e = hipFuncSetAttribute((const void*)pipe_kernel<WM, RB>,                      \
                                                     hipFuncAttributeMaxDynamicSharedMemorySize, (int)shm); \
            if (e != hipSuccess) return e;                                                                 \
            granted = shm;                                                                                 \
        }                                                                                                  \
        return launch_kernel(pipe_kernel<WM, RB>, grid, block, shm, stream, ev, a, lp, t);                 \
    }
    DT_PIPE(2, 4) DT_PIPE(2, 2) DT_PIPE(2, 1)
#undef DT_PIPE
    return hipErrorInvalidValue;
}

// LDS grant and co-residency of the persistent kernel for a plan (once per
// distinct plan: the first call sets the kernel's dynamic-LDS limit)
template <int RB>
static hipError_t pers_prepare(const PipePlan& pp, int B, bool* fits) {
    static unsigned granted = 0;  // dynamic LDS bytes allowed so far (grows only)
    const unsigned shm = (unsigned)pp.lds;
    if (shm > granted) {
        const hipError_t e =
            hipFuncSetAttribute((const void*)pers_kernel<RB>, hipFuncAttributeMaxDynamicSharedMemorySize, (int)shm);
        if (e != hipSuccess) return e;
        granted = shm;
    }
    int dev = 0, coop = 0, cus = 0, per_cu = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e == hipSuccess) e = hipDeviceGetAttribute(&coop, hipDeviceAttributeCooperativeLaunch, dev);
    if (e == hipSuccess) e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
    if (e == hipSuccess)
        e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, (const void*)pers_kernel<RB>, kPipeThreads, shm);
    if (e != hipSuccess) return e;
    *fits = coop != 0 && (long long)per_cu * cus >= (long long)pp.ng + B;
    return hipSuccess;
}

bool pers_supported(const PipePlan& pp, int B, int V, int E) {
    // (the x rows' offsets in the embedding table are 32-bit)
    if (pp.ng == 0 || B < 1 || V > kPersMaxV || (long long)V * E > 0x7fffffffLL) return false;
    bool fits = false;
    hipError_t e = hipErrorInvalidValue;
    if (pp.rb == 4) e = pers_prepare<4>(pp, B, &fits);
    else if (pp.rb == 2) e = pers_prepare<2>(pp, B, &fits);
    else if (pp.rb == 1) e = pers_prepare<1>(pp, B, &fits);
    if (e != hipSuccess) {
        (void)hipGetLastError();  // (a failed query leaves nothing pending)
        return false;
    }
    return fits;
}

hipError_t launch_pers_build(const PipeArgs& a, const PipePlan& pp, const NodeLds& lp, hipStream_t stream,
                             LaunchEvents ev, bool coop) {
    if (a.B == 0) return hipSuccess;
    // (its flags -- gflag [ng], hflag [2][B] in room for 4 B words, xflag
    // [2][B] and the error word, one run of words -- and its clock pair were
    // set by the top-M select before it)
    hipError_t e;
    if (ev.start && (e = hipEventRecord(ev.start, stream)) != hipSuccess) return e;
    PipeArgs args = a;
    NodeLds lds = lp;
    void* params[] = {&args, &lds};
    const dim3 grid(pp.ng + a.B), block(kPipeThreads);
    const void* fn = pp.rb == 4 ? (const void*)pers_kernel<4>
                   : pp.rb == 2 ? (const void*)pers_kernel<2>
                                : (const void*)pers_kernel<1>;
    e = coop ? hipLaunchCooperativeKernel(fn, grid, block, params, (unsigned)pp.lds, stream)
             : hipLaunchKernel(fn, grid, block, params, (unsigned)pp.lds, stream);
    if (e != hipSuccess) return e;
    if (ev.stop && (e = hipEventRecord(ev.stop, stream)) != hipSuccess) return e;
    return hipSuccess;
}

}  // namespace dt
