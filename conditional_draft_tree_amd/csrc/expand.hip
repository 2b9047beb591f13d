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
//   1. finish the GRU update of tree slot s from the gate sums of the
//      preceding contraction (slot 0, the root, takes h0 instead);
//   2. score slot s's children: z_j = val_j + C[idx_j] . h, z /= T, log-softmax,
//      bitonic sort by (log-prob desc, token asc) across one wave;
//   3. push slot s's best child; pop the best candidate as slot s+1 and push
//      its next-ranked sibling (lazy sibling push: the queue then holds at
//      most n entries, one per lane of a wave);
//   4. stage slot s+1's GRU input for the next contraction;
//   5. after the last step, emit the ancestor-only mask.
// The queue key orders (score desc, depth asc, parent slot asc, rank asc).
#include "dt_device.h"
#include "dt_launch.h"

namespace dt {

namespace {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

constexpr int kNodeThreads = 256;
constexpr int kRowsPerWave = kMaxM / (kNodeThreads / kWave);  // 16

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
// h is in LDS; z goes to LDS.  Every lane keeps its 16 rows' loads in flight.
template <typename T>
__device__ void correction_logits(const T* __restrict__ C, const int32_t* __restrict__ idx,
                                  const float* __restrict__ val, int M, int H, const float* hs,
                                  float* z) {
    constexpr int P = Row<T>::kPerVec;
    const int wave = threadIdx.x / kWave, lane = lane_id();
    int tok[kRowsPerWave];
    float acc[kRowsPerWave];
#pragma unroll
    for (int jj = 0; jj < kRowsPerWave; ++jj) {
        const int j = wave * kRowsPerWave + jj;
        tok[jj] = j < M ? idx[j] : -1;
        acc[jj] = 0.f;
    }
    for (int k0 = 0; k0 < H; k0 += kWave * P) {
        const int k = k0 + lane * P;
        const bool kok = k < H;
        u32x4 v[kRowsPerWave];
#pragma unroll
        for (int jj = 0; jj < kRowsPerWave; ++jj)
            v[jj] = (kok && tok[jj] >= 0)
                        ? *reinterpret_cast<const u32x4*>(C + (size_t)tok[jj] * H + k)
                        : u32x4{0u, 0u, 0u, 0u};
        float hv[P];
#pragma unroll
        for (int i = 0; i < P; ++i) hv[i] = kok ? hs[k + i] : 0.f;
#pragma unroll
        for (int jj = 0; jj < kRowsPerWave; ++jj) acc[jj] += Row<T>::dot(v[jj], hv);
    }
#pragma unroll
    for (int jj = 0; jj < kRowsPerWave; ++jj) {
        const float d = wave_sum(acc[jj]);
        const int j = wave * kRowsPerWave + jj;
        if (lane == 0 && j < M) z[j] = val[j] + d;
    }
}

// Wave 0: temperature, log-softmax over the M-slice, children sorted by
// (log-prob desc, token asc).  Lane r returns the rank-r child (key 0 when
// r >= M).
__device__ u64 sorted_children(const float* z, const int32_t* idx, int M, float temp) {
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

template <typename T>
__global__ __launch_bounds__(kNodeThreads) void node_step_kernel(NodeArgs a, int step) {
    __shared__ float hs[kMaxH];
    __shared__ float zs[kMaxM];
    __shared__ int spar[kMaxN + 1];

    const int b = blockIdx.x;
    const int lane = lane_id(), wave = threadIdx.x / kWave;
    const int S = a.n + 1;
    const size_t slot0 = (size_t)b * S;
    const int cnt = step == 0 ? 0 : a.count[b];
    // Slot `step` is expanded when it exists (every earlier pop succeeded)
    // and was staged for expansion (depth < L).
    const bool expand = step == 0 || (cnt == step && a.gru_tok[b] >= 0);
    const int depth = step == 0 ? 0 : (expand ? a.depths[slot0 + step] : 0);

    // ---- 1. hidden state of slot `step`
    if (expand) {
        float* hdst = a.hstate + (slot0 + step) * a.H;
        if (step == 0) {
            for (int k = threadIdx.x; k < a.H; k += kNodeThreads) {
                const float v = a.h0 ? a.h0[(size_t)b * a.H + k] : 0.f;
                hs[k] = v;
                hdst[k] = v;
            }
        } else {
            const float* hprev = a.hstate + (slot0 + a.gru_par[b]) * a.H;
            for (int k = threadIdx.x; k < a.H; k += kNodeThreads) {
                const float v = gru_unit_update(a.gates, a.ksplit, a.B, b, a.H, k, a.b_ih, a.b_hh,
                                                a.dtype, hprev[k]);
                hs[k] = v;
                hdst[k] = v;
            }
        }
    }
    __syncthreads();

    // ---- 2. children of slot `step` (block position = its depth)
    const size_t trow = ((size_t)b * a.L + depth) * a.M;
    if (expand)
        correction_logits<T>((const T*)a.C, a.tidx + trow, a.tval + trow, a.M, a.H, hs, zs);
    __syncthreads();
    if (wave != 0) return;

    u64 kids = 0ull;  // lane r: rank-r child of slot `step`
    if (expand) {
        kids = sorted_children(zs, a.tidx + trow, a.M, a.temp);
        const size_t crow = (slot0 + step) * kMaxM;
        if (lane < a.M) {
            a.child_tok[crow + lane] = child_tok_of(kids);
            a.child_lp[crow + lane] = child_lp_of(kids);
        }
    }

    // ---- 3. queue: push slot `step`'s best child, pop, push the sibling
    u64 q;
    int qs;
    if (step == 0) {
        q = 0ull;
        qs = 0;
        // root slot and empty slots
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
    } else {
        q = a.queue[(size_t)b * kWave + lane];
        qs = a.qsize[b];
    }
    const float score_step = step == 0 ? 0.f : a.scores[slot0 + step];
    if (expand) {
        const u64 best = shfl_u64(kids, 0);
        const u64 key = queue_key(score_step + child_lp_of(best), depth + 1, step, 0);
        if (lane == qs) q = key;
        ++qs;
    }
    uint32_t flag = step == 0 ? 0u : a.flags[b];
    int new_cnt = cnt;
    int v_par = -1;
    if (cnt == step && qs > 0) {
        const u64 top = wave_max_u64(q);
        const u64 hold = __ballot(q == top);
        const int holder = (int)__builtin_ctzll(hold);
        const u64 last = shfl_u64(q, qs - 1);
        if (lane == holder) q = last;
        if (lane == qs - 1) q = 0ull;
        --qs;

        const int pd = qk_depth(top), pp = qk_parent(top), pr = qk_rank(top);
        const float psc = qk_score(top);
        // the popped candidate's token and its next sibling's log-prob
        int ptok;
        float sib_lp = 0.f;
        const bool has_sib = pr + 1 < a.M;
        if (pp == step) {  // a child of the slot expanded just now: in registers
            ptok = child_tok_of(shfl_u64(kids, pr));
            const float l = child_lp_of(shfl_u64(kids, min(pr + 1, kWave - 1)));
            if (has_sib) sib_lp = l;
        } else {
            const size_t crow = (slot0 + pp) * kMaxM;
            ptok = a.child_tok[crow + pr];
            if (has_sib) sib_lp = a.child_lp[crow + pr + 1];
        }
        if (has_sib) {
            const float par_score = pp == 0 ? 0.f : (pp == step ? score_step : a.scores[slot0 + pp]);
            const u64 key = queue_key(par_score + sib_lp, pd, pp, pr + 1);
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
        new_cnt = v;
        v_par = pp;
        if (lane == 0) {
            a.tokens[slot0 + v] = ptok;
            a.parents[slot0 + v] = pp;
            a.depths[slot0 + v] = pd;
            a.scores[slot0 + v] = psc;
            const bool grow = pd < a.L && v < a.n;
            a.gru_tok[b] = grow ? ptok : -1;
            a.gru_par[b] = pp;
        }
    } else if (lane == 0) {
        a.gru_tok[b] = -1;
        a.gru_par[b] = 0;
    }
    a.queue[(size_t)b * kWave + lane] = q;
    if (lane == 0) {
        a.qsize[b] = qs;
        a.count[b] = new_cnt;
        a.flags[b] = flag;
    }

    // ---- 5. ancestor-only mask after the last step
    if (step == a.n - 1) {
        for (int i = lane; i < S; i += kWave) {
            int p;
            if (i == 0) p = -1;
            else if (i == step + 1 && new_cnt == step + 1) p = v_par;
            else if (i <= new_cnt) p = a.parents[slot0 + i];
            else p = -2;  // unused slot
            spar[i] = p;
        }
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "workgroup");
        for (int i = lane; i < S; i += kWave) {
            uint8_t* row = a.mask + ((size_t)b * S + i) * S;
            u64 bits_lo = 0ull;  // slots 0..63
            bool bit64 = false;  // slot 64 (only when n = 64)
            if (spar[i] != -2) {
                for (int j = i; j >= 0; j = j == 0 ? -1 : spar[j]) {
                    if (j < 64) bits_lo |= 1ull << j;
                    else bit64 = true;
                }
            }
            for (int j = 0; j < S; ++j)
                row[j] = (uint8_t)(j < 64 ? ((bits_lo >> j) & 1ull) : (bit64 ? 1 : 0));
        }
    }
}

template <typename T>
__global__ __launch_bounds__(kNodeThreads) void correct_kernel(const int32_t* tidx, const float* tval,
                                                               const T* C, const float* h,
                                                               const int32_t* pos, int32_t* tok_out,
                                                               float* lp_out, int L, int H, int M,
                                                               float temp) {
    __shared__ float hs[kMaxH];
    __shared__ float zs[kMaxM];
    const int b = blockIdx.x;
    for (int k = threadIdx.x; k < H; k += kNodeThreads) hs[k] = h[(size_t)b * H + k];
    __syncthreads();
    const size_t trow = ((size_t)b * L + pos[b]) * M;
    correction_logits<T>(C, tidx + trow, tval + trow, M, H, hs, zs);
    __syncthreads();
    if (threadIdx.x >= kWave) return;
    const u64 kids = sorted_children(zs, tidx + trow, M, temp);
    const int lane = lane_id();
    if (lane < M) {
        tok_out[(size_t)b * M + lane] = child_tok_of(kids);
        lp_out[(size_t)b * M + lane] = child_lp_of(kids);
    }
}

}  // namespace

hipError_t launch_node_step(const NodeArgs& a, int step, hipStream_t stream) {
    if (a.B == 0) return hipSuccess;
    if (a.dtype == 1)
        node_step_kernel<bf16_t><<<a.B, kNodeThreads, 0, stream>>>(a, step);
    else
        node_step_kernel<float><<<a.B, kNodeThreads, 0, stream>>>(a, step);
    return hipGetLastError();
}

hipError_t launch_correct(const int32_t* tidx, const float* tval, const void* C, const float* h,
                          const int32_t* pos, int32_t* tok_sorted, float* lp_sorted, int B, int L,
                          int H, int M, int dtype, float temp, hipStream_t stream) {
    if (B == 0) return hipSuccess;
    if (dtype == 1)
        correct_kernel<bf16_t><<<B, kNodeThreads, 0, stream>>>(tidx, tval, (const bf16_t*)C, h, pos,
                                                               tok_sorted, lp_sorted, L, H, M, temp);
    else
        correct_kernel<float><<<B, kNodeThreads, 0, stream>>>(tidx, tval, (const float*)C, h, pos,
                                                              tok_sorted, lp_sorted, L, H, M, temp);
    return hipGetLastError();
}

}  // namespace dt
