// accept.hip -- greedy (temperature 0) acceptance of verified draft trees,
// one wave per request.
//
// After the target model has scored every node of a tree in one forward
// pass, serial greedy decoding agrees with the draft along one root path:
// at the current node (first the root) the target's greedy token selects
// the child that carries it, and the walk ends at a node with no such child;
// the target's token there is emitted as well ([captcha] "Methodology --
// deep read": the longest accepted root-to-leaf path of one verification
// pass; [gist] "Résultats expérimentaux -- Absence de perte": the output
// equals serial greedy decoding).
#include "dt_device.h"
#include "dt_launch.h"

namespace dt {

namespace {

// Slots 0..n of request b, n <= 64: lane l holds slots l and l + 64 (the
// latter exists only when n = 64).  Each step is one ballot over the slots;
// the walk cannot revisit a node (a node's only parent is the node before
// it on the walk, and slot 0 is never a child), so it ends within count
// steps; the loop bound n only guards malformed input.
__global__ __launch_bounds__(kWave) void accept_greedy_kernel(const int32_t* __restrict__ tokens,
                                                              const int32_t* __restrict__ parents,
                                                              const int32_t* __restrict__ count,
                                                              const int32_t* __restrict__ target, int n,
                                                              int32_t* path, int32_t* accepted,
                                                              int32_t* bonus) {
    const int b = blockIdx.x, lane = lane_id();
    const int S = n + 1;
    const size_t row = (size_t)b * S;
    const int cnt = min(max(count[b], 0), n);
    const int s0 = lane, s1 = lane + kWave;
    const bool v0 = s0 < S, v1 = s1 < S;
    const int tk0 = v0 ? tokens[row + s0] : -1, pa0 = v0 ? parents[row + s0] : -1;
    const int tk1 = v1 ? tokens[row + s1] : -1, pa1 = v1 ? parents[row + s1] : -1;
    const int tg0 = v0 ? target[row + s0] : -1, tg1 = v1 ? target[row + s1] : -1;
    // children candidates: slots 1..count
    const bool in0 = s0 >= 1 && s0 <= cnt, in1 = s1 >= 1 && s1 <= cnt;
    int u = 0, k = 0, mine = -1;  // mine: path entry `lane` (k <= n - 1 <= 63)
    int tu = __builtin_amdgcn_readlane(tg0, 0);  // the target's token at the current node
    while (k < n) {
        const u64 m0 = __ballot(in0 && pa0 == u && tk0 == tu);
        const u64 m1 = __ballot(in1 && pa1 == u && tk1 == tu);
        if (m0 == 0ull && m1 == 0ull) break;
        u = m0 ? (int)__builtin_ctzll(m0) : kWave + (int)__builtin_ctzll(m1);  // lowest slot
        if (lane == k) mine = u;
        ++k;
        tu = u < kWave ? __builtin_amdgcn_readlane(tg0, u) : __builtin_amdgcn_readlane(tg1, u - kWave);
    }
    if (v0) path[row + s0] = mine;
    if (v1) path[row + s1] = -1;  // entry 64: at most n = 64 tokens are accepted (entries 0..63)
    if (lane == 0) {
        accepted[b] = k;
        bonus[b] = tu;
    }
}

}  // namespace

hipError_t launch_accept_greedy(const int32_t* tokens, const int32_t* parents, const int32_t* count,
                                const int32_t* target, int B, int n, int32_t* path, int32_t* accepted,
                                int32_t* bonus, hipStream_t stream, LaunchEvents ev) {
    if (B == 0) return hipSuccess;
    return launch_kernel(accept_greedy_kernel, dim3(B), dim3(kWave), 0, stream, ev, tokens, parents, count,
                         target, n, path, accepted, bonus);
}

}  // namespace dt
