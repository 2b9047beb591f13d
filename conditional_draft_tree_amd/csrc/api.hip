// api.hip -- the C ABI declared in include/dtree.h: argument checks, the
// workspace plan and the launch sequence of one build.
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <algorithm>
#include <mutex>
#include <string>
#include <vector>

#include "../../include/dtree.h"
#include "dt_launch.h"

// dt_build_noalloc's scratch (see scratch_on below): file scope, one copy per
// device, held until the process ends.
constexpr size_t kScratchBytes = (size_t)32 << 20;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

namespace {

using dt::u64;

constexpr size_t kAlign = 256;
size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

thread_local char g_create_error[512] = "";

struct Layout {
    size_t partial, tidx, tval, hstate, hsplit, gpart, gru_tok, gru_par, child_tok, child_lp, ckey, queue, nidx, nval,
        rstate, xpack, hpack, hprev, tail, tail_part, wpack;
    // fused expansion only (sizes 0 otherwise)
    size_t p_gi, p_gh, p_hstate, p_exp, p_done, p_active, p_xpack1, p_hpack1, p_xtok, p_hslot;
    size_t total;
};

struct Marker {
    // 'K'/'T' begin/end of the top-M select kernel, 'M' after the top-M merge,
    // 'g'/'G' begin/end of a gate contraction, 'n'/'N' of a node step, 'E'
    // end of the call; 'a'/'A' begin/end of a dt_accept_greedy kernel.  A
    // stage's time is the span from the preceding marker, or, where `clock`
    // >= 0 (the persistent expansion), the device-clock span that the launch
    // wrote into slot `clock` of the handle's clock buffer.
    char tag;
    hipEvent_t ev;
    int clock = -1;
};

}  // namespace

struct dt_handle {
    dt_config cfg;
    int nseg;    // top-M segments per row
    int ksplit;    // K ranges of the gate contraction
    int ksplit_f;  // of its recurrent part alone (folded input projection)
    dt::NodeLds lds;
    dt::PipePlan pp;  // fused expansion plan (pp.ng = 0: stepped)
    int pipe_T;       // launches of a fused call
    int pers = -1;    // the device holds the persistent grid: 1 yes, 0 no, -1 not checked yet
    int32_t last_mode;  // expansion of the last dt_build call (before any: the configured one)
    Layout lay;
    Layout lay_na;  // dt_build_noalloc's use of the static scratch (no weight-tile copy)
    std::string err;
    // timing
    int tlevel = 0;
    int tcapacity = 0;
    std::vector<std::vector<Marker>> calls;
    std::vector<hipEvent_t> pool;
    size_t pool_used = 0;
    unsigned long long* tclock = nullptr;  // [capacity][2] device clock of persistent launches (level 2)
    int tclock_cap = 0;
};

namespace {

dt_status fail(dt_handle* h, dt_status s, const char* fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    if (h)
        h->err = buf;
    else
        snprintf(g_create_error, sizeof g_create_error, "%s", buf);
    return s;
}

dt_status hip_fail(dt_handle* h, hipError_t e, const char* what) {
    return fail(h, DT_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

// log2(e) / T (T = 1 when the temperature is 0): the top-M select sums
// 2^(x * this) for the full-vocabulary tail
float tail_scale(const dt_config& c) {
    return 1.4426950408889634f / (c.temperature > 0.f ? c.temperature : 1.f);
}

// ksplit: the larger of the two; wtiles: room for the weights in operand tiles;
// pp: the fused expansion's plan (pp.ng = 0: none), pT its launches per call
Layout plan_layout(const dt_config& c, int nseg, int ksplit, bool wtiles = true, dt::PipePlan pp = {},
                   int pT = 0) {
    Layout l{};
    const size_t B = c.B, L = c.L, M = c.M, S = (size_t)c.n + 1, H = c.H;
    size_t off = 0;
    auto take = [&](size_t bytes) {
        size_t at = off;
        off = align_up(off + bytes);
        return at;
    };
    l.partial = take(B * L * (size_t)nseg * 64 * sizeof(u64));
    l.tidx = take(B * L * M * 4);
    l.tval = take(B * L * M * 4);
    l.hstate = take(c.dtype == DT_F32 ? B * S * H * 4 : 0);  // the bf16 path keeps bf16 parts only
    l.hsplit = take(c.dtype == DT_BF16 ? B * S * 3 * H * 2 : 0);
    l.gpart = take((size_t)ksplit * B * dt::kGateSlotsHost * H * 4);
    l.gru_tok = take(B * 4);
    l.gru_par = take(B * 4);
    l.child_tok = take(B * S * 64 * 4);
    l.child_lp = take(B * S * 64 * 4);
    l.ckey = take(B * S * 64 * sizeof(u64));
    l.queue = take(B * 64 * sizeof(u64));
    l.rstate = take(B * dt::kStateWords * 4);
    l.nidx = take(B * 64 * 4);
    l.xpack = take(c.dtype == DT_BF16 ? (size_t)dt::pack_rows(c.B) * c.E * 2 : 0);
    l.hpack = take(c.dtype == DT_BF16 ? (size_t)dt::pack_rows(c.B) * 3 * H * 2 : 0);
    l.hprev = take(c.dtype == DT_BF16 ? B * H * 4 : 0);
    l.nval = take(B * 64 * 4);
    l.tail = take(B * L * 4);                          // full-vocabulary mode: tail_lse per row
    l.tail_part = take(B * L * (size_t)nseg * 2 * 4);  // its per-segment (m, s) sums
    l.wpack = take(wtiles && c.dtype == DT_BF16 ? (size_t)3 * H * (c.E + c.H) * 2 : 0);  // weights in operand tiles
    const bool fp = pp.ng > 0;
    l.p_gi = take(fp ? 2 * (size_t)pp.ksx * B * 3 * H * 4 : 0);  // x-part gate sums by launch parity
    l.p_gh = take(fp ? B * S * (size_t)pp.ksh * 3 * H * 4 : 0);  // h-part gate sums per slot
    l.p_hstate = take(fp ? B * S * H * 4 : 0);        // binary32 state per slot
    l.p_exp = take(fp ? B * S * 4 : 0);               // launch that expanded each slot
    // per-launch counters, then each slice's flags and error word
    l.p_done = take(fp ? ((size_t)pT + (size_t)dt::pers_slices(c.B) * dt::pers_flag_words(pp, dt::pers_slice_b(c.B))) * 4
                       : 0);
    l.p_active = take(fp ? (size_t)2 * pT * 4 : 0);
    l.p_xpack1 = take(fp ? (size_t)dt::pack_rows(c.B) * c.E * 2 : 0);  // parity-1 activations
    l.p_hpack1 = take(fp ? (size_t)dt::pack_rows(c.B) * 3 * H * 2 : 0);
    l.p_xtok = take(fp ? 2 * B * 4 : 0);
    l.p_hslot = take(fp ? 2 * B * 4 : 0);
    l.total = off;
    return l;
}

bool misaligned(const void* p) { return p && ((uintptr_t)p % 16) != 0; }

// An error that earlier asynchronous HIP work left on this host thread (a
// failed launch, an error reported since) is returned, and cleared, before
// anything is enqueued, so that it is not blamed on a later call that
// succeeds.  Called after argument validation, which makes no HIP call.
dt_status pending_error(dt_handle* h) {
    const hipError_t e = hipGetLastError();
    return e == hipSuccess ? DT_OK : hip_fail(h, e, "HIP error pending from earlier asynchronous work");
}

// dt_build_noalloc's scratch: a file-scope device array, one copy on each GPU
// the library runs on, held until the process ends.  On the host, `scratch`
// names a stand-in, not a device address: host code uses only the address
// that hipGetSymbolAddress returns for each device (kept in g_scratch).
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch[kMaxDevices] = {};

// The scratch address on `stream`'s device, which must be the calling
// thread's current device (looked up once per device, with it current).
dt_status scratch_on(dt_handle* h, hipStream_t stream, void** out) {
    int cur = -1, dev = -1;
    hipError_t e = hipGetDevice(&cur);
    if (e != hipSuccess) return hip_fail(h, e, "hipGetDevice");
    e = hipStreamGetDevice(stream, &dev);
    if (e != hipSuccess) return hip_fail(h, e, "hipStreamGetDevice");
    if (dev != cur)
        return fail(h, DT_ERR_INVALID_ARG, "dt_build_noalloc: the stream is on device %d, the current device is %d",
                    dev, cur);
    if (dev < 0 || dev >= kMaxDevices)
        return fail(h, DT_ERR_UNSUPPORTED, "dt_build_noalloc: device %d beyond %d", dev, kMaxDevices);
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch[dev]) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return hip_fail(h, e, "hipGetSymbolAddress(scratch)");
        if (!p || (uintptr_t)p % kAlign)
            return fail(h, DT_ERR_HIP, "dt_build_noalloc: scratch address %p is not %zu-byte aligned", p, kAlign);
        g_scratch[dev] = p;
    }
    *out = g_scratch[dev];
    return DT_OK;
}

dt_status check_ws(dt_handle* h, void* ws, size_t bytes) {
    if (h->lay.total == 0) return DT_OK;
    if (!ws) return fail(h, DT_ERR_WORKSPACE, "workspace is NULL (need %zu bytes)", h->lay.total);
    if (bytes < h->lay.total)
        return fail(h, DT_ERR_WORKSPACE, "workspace has %zu bytes, need %zu", bytes, h->lay.total);
    if ((uintptr_t)ws % kAlign)
        return fail(h, DT_ERR_WORKSPACE, "workspace must be %zu-byte aligned", kAlign);
    return DT_OK;
}

hipEvent_t take_event(dt_handle* h) {
    if (h->pool_used == h->pool.size()) {
        hipEvent_t e;
        if (hipEventCreate(&e) != hipSuccess) return nullptr;
        h->pool.push_back(e);
    }
    return h->pool[h->pool_used++];
}

// Record a timing marker of the current call (level >= need).
hipError_t mark(dt_handle* h, std::vector<Marker>* call, int need, char tag, hipStream_t st) {
    if (!call || h->tlevel < need) return hipSuccess;
    hipEvent_t e = take_event(h);
    if (!e) return hipErrorOutOfMemory;
    call->push_back({tag, e});
    return hipEventRecord(e, st);
}

// Begin/end markers (tags t0, t1) of the next kernel of the current call
// (level >= need): `ev` receives two events that the launch itself records.
// Below the level, `ev` is cleared and the launch is untimed.
hipError_t kernel_marks(dt_handle* h, std::vector<Marker>* call, int need, char t0, char t1,
                        dt::LaunchEvents* ev) {
    *ev = dt::LaunchEvents{};
    if (!call || h->tlevel < need) return hipSuccess;
    hipEvent_t e0 = take_event(h), e1 = take_event(h);
    if (!e0 || !e1) return hipErrorOutOfMemory;
    call->push_back({t0, e0});
    call->push_back({t1, e1});
    ev->start = e0;
    ev->stop = e1;
    return hipSuccess;
}

}  // namespace

extern "C" {

const char* dt_status_string(dt_status s) {
    int32_t v;  // any int from a C caller: read it as one (see dt_create)
    memcpy(&v, &s, sizeof v);
    switch (v) {
        case DT_OK: return "ok";
        case DT_ERR_INVALID_ARG: return "invalid argument";
        case DT_ERR_UNSUPPORTED: return "unsupported configuration";
        case DT_ERR_WORKSPACE: return "workspace missing or too small";
        case DT_ERR_HIP: return "HIP runtime error";
    }
    return "unknown status";
}

const char* dt_last_error(const dt_handle* h) { return h ? h->err.c_str() : g_create_error; }

dt_status dt_create(const dt_config* cfg, dt_handle** out) {
    if (!out) return fail(nullptr, DT_ERR_INVALID_ARG, "out is NULL");
    *out = nullptr;
    if (!cfg) return fail(nullptr, DT_ERR_INVALID_ARG, "cfg is NULL");
    // the dtype field arrives from C callers as any int: read it as one, since
    // a value outside the enumerators is not a valid dt_dtype in C++
    static_assert(sizeof(dt_dtype) == sizeof(int32_t), "dt_dtype is stored as a 32-bit int");
    int32_t dtype_raw;
    memcpy(&dtype_raw, &cfg->dtype, sizeof dtype_raw);
    if (dtype_raw != (int32_t)DT_F32 && dtype_raw != (int32_t)DT_BF16)
        return fail(nullptr, DT_ERR_INVALID_ARG, "dtype %d is neither DT_F32 nor DT_BF16", (int)dtype_raw);
    const dt_config c = *cfg;
    if (c.B < 0 || c.L < 1 || c.V < 1 || c.E < 1 || c.H < 1 || c.M < 1 || c.n < 1)
        return fail(nullptr, DT_ERR_INVALID_ARG,
                    "sizes must be positive (B >= 0): B=%d L=%d V=%d E=%d H=%d M=%d n=%d", c.B, c.L,
                    c.V, c.E, c.H, c.M, c.n);
    if (c.M > c.V) return fail(nullptr, DT_ERR_INVALID_ARG, "M=%d exceeds V=%d", c.M, c.V);
    if (!(c.temperature >= 0.f) || !(c.near_tie_eps >= 0.f))
        return fail(nullptr, DT_ERR_INVALID_ARG, "temperature and near_tie_eps must be >= 0");
    if (c.full_vocab != 0 && c.full_vocab != 1)
        return fail(nullptr, DT_ERR_INVALID_ARG, "full_vocab must be 0 or 1 (got %d)", (int)c.full_vocab);
    if (c.expand < DT_EXPAND_AUTO || c.expand > DT_EXPAND_RESIDENT)
        return fail(nullptr, DT_ERR_INVALID_ARG, "expand must be 0, 1, 2 or 3 (got %d)", (int)c.expand);
    if (c.M > 64) return fail(nullptr, DT_ERR_UNSUPPORTED, "M=%d > 64 (one candidate per lane)", c.M);
    if (c.n > 64) return fail(nullptr, DT_ERR_UNSUPPORTED, "n=%d > 64 (queue of one wave)", c.n);
    if (c.L > 64) return fail(nullptr, DT_ERR_UNSUPPORTED, "L=%d > 64", c.L);
    if (c.H > 4096) return fail(nullptr, DT_ERR_UNSUPPORTED, "H=%d > 4096", c.H);
    if (c.dtype == DT_BF16 && (c.E % 32 || c.H % 32))
        return fail(nullptr, DT_ERR_UNSUPPORTED, "bf16 needs E %% 32 == 0 and H %% 32 == 0 (E=%d H=%d)",
                    c.E, c.H);
    if (c.dtype == DT_F32 && (c.E % 4 || c.H % 4))
        return fail(nullptr, DT_ERR_UNSUPPORTED, "f32 needs E %% 4 == 0 and H %% 4 == 0 (E=%d H=%d)",
                    c.E, c.H);
    if ((long long)c.B * c.L * c.V > (1ll << 40))
        return fail(nullptr, DT_ERR_UNSUPPORTED, "B*L*V too large");
    const dt::NodeLds lds = dt::node_lds_plan(c.L, c.M, c.n, c.H);
    if (lds.bytes > 65536)
        return fail(nullptr, DT_ERR_UNSUPPORTED,
                    "per-request state needs %zu bytes of LDS (> 64 KiB): lower L*M, n or H",
                    lds.bytes);
    const int nseg = dt::topm_segments(c.B * c.L, c.V);
    const size_t seg_bytes = ((size_t)c.V + nseg - 1) / nseg * (c.dtype == DT_BF16 ? 2 : 4);
    if (seg_bytes > (1u << 30))  // the select addresses a segment with 32-bit byte offsets
        return fail(nullptr, DT_ERR_UNSUPPORTED, "top-M segment of %zu bytes exceeds 1 GiB", seg_bytes);
    dt_handle* h = new dt_handle();
    h->cfg = c;
    h->nseg = nseg;
    h->ksplit = dt::gru_ksplit(c.B, c.E, c.H, (int)c.dtype);
    h->ksplit_f = dt::gru_ksplit(c.B, 0, c.H, (int)c.dtype);
    h->lds = lds;
    h->pp = dt::PipePlan{};
    h->pipe_T = 0;
    if (c.expand == DT_EXPAND_FUSED && c.B > dt::kPipeSliceB) {
        delete h;
        return fail(nullptr, DT_ERR_UNSUPPORTED, "one launch per step needs B <= %d", dt::kPipeSliceB);
    }
    // more requests than one grid holds: the persistent launch in slices (with
    // the plan of one) only when asked for -- on deep chains its requests wait
    // inside the steps, and the slices run one after another
    if (c.dtype == DT_BF16 && c.expand != DT_EXPAND_STEPPED &&
        (c.B <= dt::kPipeSliceB || c.expand == DT_EXPAND_PERSISTENT || c.expand == DT_EXPAND_RESIDENT)) {
        h->pp = dt::pipe_plan(dt::pers_slice_b(c.B), c.L, c.E, c.H, c.M, c.n);
        h->pipe_T = c.n + 2;
    }
    if ((c.expand == DT_EXPAND_FUSED || c.expand == DT_EXPAND_PERSISTENT || c.expand == DT_EXPAND_RESIDENT) &&
        h->pp.ng == 0) {
        delete h;
        return fail(nullptr, DT_ERR_UNSUPPORTED,
                    "fused expansion needs bf16, H <= 1024 and E, H multiples of 32");
    }
    h->last_mode = h->pp.ng == 0                   ? DT_EXPAND_STEPPED
                   : c.expand == DT_EXPAND_FUSED      ? DT_EXPAND_FUSED
                   : c.expand == DT_EXPAND_PERSISTENT ? DT_EXPAND_PERSISTENT
                                                      : DT_EXPAND_RESIDENT;
    h->lay = plan_layout(c, h->nseg, std::max(h->ksplit, h->ksplit_f), true, h->pp, h->pipe_T);
    h->lay_na = plan_layout(c, h->nseg, h->ksplit, /*wtiles=*/false);
    *out = h;
    return DT_OK;
}

void dt_destroy(dt_handle* h) {
    if (!h) return;
    for (hipEvent_t e : h->pool) (void)hipEventDestroy(e);
    if (h->tclock) (void)hipFree(h->tclock);
    delete h;
}

size_t dt_workspace_bytes(const dt_handle* h) { return h ? h->lay.total : 0; }

int32_t dt_expand_mode(const dt_handle* h) {
    if (!h) return -1;
    return h->last_mode;
}

dt_status dt_timing_enable(dt_handle* h, int level, int capacity) {
    if (!h) return DT_ERR_INVALID_ARG;
    if (level < 0 || level > 2 || capacity < 0)
        return fail(h, DT_ERR_INVALID_ARG, "timing level must be 0..2 and capacity >= 0");
    h->calls.clear();
    h->pool_used = 0;
    h->tlevel = level;
    h->tcapacity = level ? capacity : 0;
    // the device-clock slots of the persistent expansion (level 2)
    if (level == 2 && capacity > h->tclock_cap) {
        if (h->tclock) (void)hipFree(h->tclock);
        h->tclock = nullptr;
        h->tclock_cap = 0;
        const hipError_t e = hipMalloc((void**)&h->tclock, (size_t)capacity * 2 * sizeof(unsigned long long));
        if (e != hipSuccess) {
            h->tlevel = 0;
            h->tcapacity = 0;
            return hip_fail(h, e, "timing clock buffer");
        }
        h->tclock_cap = capacity;
    }
    return DT_OK;
}

dt_status dt_timing_read(dt_handle* h, int stage, float* ms, int max, int* n_out) {
    if (!h || !n_out || (max > 0 && !ms)) return h ? fail(h, DT_ERR_INVALID_ARG, "null output") : DT_ERR_INVALID_ARG;
    if (stage < 0 || stage > 8) return fail(h, DT_ERR_INVALID_ARG, "stage must be 0..8");
    // the persistent launches' device-clock spans, when any call recorded one
    std::vector<unsigned long long> clk;
    for (const auto& call : h->calls)
        for (const Marker& m : call)
            if (m.clock >= 0 && clk.empty()) {
                clk.resize((size_t)h->tclock_cap * 2);
                const hipError_t e = hipMemcpy(clk.data(), h->tclock, clk.size() * sizeof(unsigned long long),
                                               hipMemcpyDeviceToHost);
                if (e != hipSuccess) return hip_fail(h, e, "timing clock read");
            }
    int n = 0;
    for (const auto& call : h->calls) {
        float sum = 0.f;
        bool any = false;
        for (size_t i = 1; i < call.size(); ++i) {
            const char tag = call[i].tag;
            bool hit = (stage == 0 && tag == 'T') || (stage == 1 && tag == 'M') ||
                       (stage == 2 && tag == 'G') || (stage == 3 && tag == 'N') ||
                       (stage == 5 && tag == 'G') || (stage == 6 && tag == 'A') ||
                       ((stage == 7 || stage == 8) && tag == 'P');
            if (!hit) continue;
            float t = 0.f;
            if (call[i].clock >= 0) {  // (the device's constant 100 MHz clock)
                const unsigned long long t0 = clk[2 * call[i].clock], t1 = clk[2 * call[i].clock + 1];
                t = t1 > t0 ? (float)((double)(t1 - t0) * 1e-5) : 0.f;
            } else {
                hipError_t e = hipEventElapsedTime(&t, call[i - 1].ev, call[i].ev);
                if (e != hipSuccess) return hip_fail(h, e, "hipEventElapsedTime");
            }
            if (stage == 5 || stage == 8) {
                if (n < max) ms[n] = t;
                ++n;
            } else {
                sum += t;
                any = true;
            }
        }
        if (stage == 4 && call.size() >= 2) {
            float t = 0.f;
            hipError_t e = hipEventElapsedTime(&t, call.front().ev, call.back().ev);
            if (e != hipSuccess) return hip_fail(h, e, "hipEventElapsedTime");
            sum = t;
            any = true;
        }
        if (stage != 5 && stage != 8 && any) {
            if (n < max) ms[n] = sum;
            ++n;
        }
    }
    *n_out = n;
    return DT_OK;
}

dt_status dt_topm(dt_handle* h, void* ws, size_t ws_bytes, const void* base, int32_t* idx, float* val,
                  void* stream) {
    if (!h) return DT_ERR_INVALID_ARG;
    const dt_config& c = h->cfg;
    if (c.B == 0) return DT_OK;
    if (!base || !idx || !val) return fail(h, DT_ERR_INVALID_ARG, "dt_topm: null pointer");
    if (misaligned(base) || misaligned(idx) || misaligned(val))
        return fail(h, DT_ERR_INVALID_ARG, "dt_topm: buffers must be 16-byte aligned");
    dt_status s = check_ws(h, ws, ws_bytes);
    if (s || (s = pending_error(h))) return s;
    hipError_t e = dt::launch_topm(base, (int)c.dtype, c.B * c.L, c.V, h->nseg,
                                   (u64*)((char*)ws + h->lay.partial), c.M, idx, val,
                                   (hipStream_t)stream);
    return e == hipSuccess ? DT_OK : hip_fail(h, e, "dt_topm launch");
}

dt_status dt_topm_tail(dt_handle* h, void* ws, size_t ws_bytes, const void* base, int32_t* idx, float* val,
                       float* tail, void* stream) {
    if (!h) return DT_ERR_INVALID_ARG;
    const dt_config& c = h->cfg;
    if (c.B == 0) return DT_OK;
    if (!base || !idx || !val || !tail) return fail(h, DT_ERR_INVALID_ARG, "dt_topm_tail: null pointer");
    if (misaligned(base) || misaligned(idx) || misaligned(val))
        return fail(h, DT_ERR_INVALID_ARG, "dt_topm_tail: buffers must be 16-byte aligned");
    dt_status s = check_ws(h, ws, ws_bytes);
    if (s || (s = pending_error(h))) return s;
    hipError_t e = dt::launch_topm(base, (int)c.dtype, c.B * c.L, c.V, h->nseg,
                                   (u64*)((char*)ws + h->lay.partial), c.M, idx, val, (hipStream_t)stream,
                                   dt::LaunchEvents{}, tail_scale(c), tail,
                                   (float*)((char*)ws + h->lay.tail_part));
    return e == hipSuccess ? DT_OK : hip_fail(h, e, "dt_topm_tail launch");
}

dt_status dt_gru_step(dt_handle* h, void* ws, size_t ws_bytes, const void* x, const float* h_in,
                      const void* W_ih, const void* W_hh, const void* b_ih, const void* b_hh,
                      float* h_out, void* stream) {
    if (!h) return DT_ERR_INVALID_ARG;
    const dt_config& c = h->cfg;
    if (c.B == 0) return DT_OK;
    if (!x || !h_in || !W_ih || !W_hh || !h_out)
        return fail(h, DT_ERR_INVALID_ARG, "dt_gru_step: null pointer");
    if (misaligned(x) || misaligned(h_in) || misaligned(W_ih) || misaligned(W_hh) || misaligned(h_out))
        return fail(h, DT_ERR_INVALID_ARG, "dt_gru_step: buffers must be 16-byte aligned");
    if ((const void*)h_out == (const void*)h_in)
        return fail(h, DT_ERR_INVALID_ARG, "dt_gru_step: h_out must not alias h");
    dt_status s = check_ws(h, ws, ws_bytes);
    if (s || (s = pending_error(h))) return s;
    hipStream_t st = (hipStream_t)stream;
    char* w = (char*)ws;
    dt::GruGatesArgs g{};
    g.xpack = (uint16_t*)(w + h->lay.xpack);
    g.hpack = (uint16_t*)(w + h->lay.hpack);
    g.x = x;
    g.xtok = nullptr;
    g.hf = h_in;
    g.hrows = 1;
    g.hsel = nullptr;
    g.W_ih = W_ih;
    g.W_hh = W_hh;
    g.partial = (float*)(w + h->lay.gpart);
    g.B = c.B;
    g.E = c.E;
    g.H = c.H;
    g.ksplit = h->ksplit;
    g.dtype = (int)c.dtype;
    hipError_t e = hipSuccess;
    if (c.dtype == DT_BF16)
        e = dt::launch_pack((const uint16_t*)x, h_in, (uint16_t*)g.xpack, (uint16_t*)g.hpack, c.B, c.E, c.H, st);
    if (e != hipSuccess) return hip_fail(h, e, "dt_gru_step packing launch");
    e = dt::launch_gru_gates(g, st);
    if (e != hipSuccess) return hip_fail(h, e, "dt_gru_step contraction launch");
    e = dt::launch_finalize(g.partial, g.ksplit, b_ih, b_hh, h_in, h_out, c.B, c.H, (int)c.dtype, st);
    return e == hipSuccess ? DT_OK : hip_fail(h, e, "dt_gru_step update launch");
}

dt_status dt_correct(dt_handle* h, const int32_t* idx, const float* val, const void* C,
                     const float* h_in, const int32_t* pos, int32_t* tok_sorted, float* logp_sorted,
                     void* stream) {
    if (!h) return DT_ERR_INVALID_ARG;
    const dt_config& c = h->cfg;
    if (c.B == 0) return DT_OK;
    if (!idx || !val || !C || !h_in || !pos || !tok_sorted || !logp_sorted)
        return fail(h, DT_ERR_INVALID_ARG, "dt_correct: null pointer");
    if (misaligned(C) || misaligned(h_in))
        return fail(h, DT_ERR_INVALID_ARG, "dt_correct: C and h must be 16-byte aligned");
    if (dt_status s = pending_error(h)) return s;
    hipError_t e = dt::launch_correct(idx, val, C, h_in, pos, tok_sorted, logp_sorted, c.B, c.L, c.H,
                                      c.M, (int)c.dtype, c.temperature, (hipStream_t)stream);
    return e == hipSuccess ? DT_OK : hip_fail(h, e, "dt_correct launch");
}

dt_status dt_accept_greedy(dt_handle* h, const int32_t* tokens, const int32_t* parents, const int32_t* count,
                           const int32_t* target, int32_t* path, int32_t* accepted, int32_t* bonus,
                           void* stream) {
    if (!h) return DT_ERR_INVALID_ARG;
    const dt_config& c = h->cfg;
    if (c.B == 0) return DT_OK;
    if (!tokens || !parents || !count || !target || !path || !accepted || !bonus)
        return fail(h, DT_ERR_INVALID_ARG, "dt_accept_greedy: null pointer");
    if (dt_status s = pending_error(h)) return s;
    std::vector<Marker>* call = nullptr;
    if (h->tlevel > 0 && (int)h->calls.size() < h->tcapacity) {
        h->calls.emplace_back();
        call = &h->calls.back();
    }
    dt::LaunchEvents ev{};
    hipError_t e = kernel_marks(h, call, 1, 'a', 'A', &ev);
    if (e != hipSuccess) return hip_fail(h, e, "timing event");
    e = dt::launch_accept_greedy(tokens, parents, count, target, c.B, c.n, path, accepted, bonus,
                                 (hipStream_t)stream, ev);
    return e == hipSuccess ? DT_OK : hip_fail(h, e, "dt_accept_greedy launch");
}

}  // extern "C"

namespace {
// table: the folded input projection [V, 3H] (dt_build_folded; emb, W_ih and
// b_ih are then unused), or NULL.  noalloc: the workspace is the device's
// static scratch (ws is ignored) and the weights are read in place.
dt_status build_impl(bool marginal, dt_handle* h, void* ws, size_t ws_bytes, const void* base, const void* emb,
                   const void* W_ih, const void* W_hh, const void* b_ih, const void* b_hh,
                   const void* C, const float* h0, int32_t* tokens, int32_t* parents, int32_t* depths,
                   float* scores, uint8_t* mask, int32_t* count, uint32_t* flags, void* stream,
                   const float* table = nullptr, bool noalloc = false) {
    if (!h) return DT_ERR_INVALID_ARG;
    const dt_config& c = h->cfg;
    if (c.B == 0) return DT_OK;
    if (!base || !tokens || !parents || !depths || !scores || !mask || !count || !flags)
        return fail(h, DT_ERR_INVALID_ARG, "dt_build: null pointer");
    if (!marginal && !table && (!emb || !W_ih || !W_hh || !C))
        return fail(h, DT_ERR_INVALID_ARG, "dt_build: null pointer (only b_ih, b_hh, h0 may be NULL)");
    if (table && (!W_hh || !C))
        return fail(h, DT_ERR_INVALID_ARG, "dt_build_folded: null pointer (only b_hh, h0 may be NULL)");
    if (misaligned(table))
        return fail(h, DT_ERR_INVALID_ARG, "dt_build_folded: the table must be 16-byte aligned");
    if (misaligned(base) || misaligned(emb) || misaligned(W_ih) || misaligned(W_hh) || misaligned(C) ||
        misaligned(h0) || misaligned(b_ih) || misaligned(b_hh))
        return fail(h, DT_ERR_INVALID_ARG, "dt_build: matrices must be 16-byte aligned");
    hipStream_t st = (hipStream_t)stream;
    dt_status s = DT_OK;
    if (noalloc) {
        if (h->lay_na.total > kScratchBytes)
            return fail(h, DT_ERR_UNSUPPORTED, "dt_build_noalloc: needs %zu bytes of scratch, the maximum is %zu",
                        h->lay_na.total, kScratchBytes);
        if ((s = pending_error(h)) || (s = scratch_on(h, st, &ws))) return s;
    } else if ((s = check_ws(h, ws, ws_bytes)) || (s = pending_error(h))) {
        return s;
    }
    char* w = (char*)ws;
    const Layout& L = noalloc ? h->lay_na : h->lay;

    std::vector<Marker>* call = nullptr;
    if (h->tlevel > 0 && (int)h->calls.size() < h->tcapacity) {
        h->calls.emplace_back();
        call = &h->calls.back();
    }
    hipError_t e;
#define DT_TRY(expr, what)                                 \
    do {                                                   \
        e = (expr);                                        \
        if (e != hipSuccess) return hip_fail(h, e, what);  \
    } while (0)

    // the expansion's mode, decided before anything is enqueued: the
    // persistent launch where the device holds its grid and the stream is
    // not being captured, else one launch per step (fused), or the stepped
    // launches.  The persistent launch's flags and clock pair are set by the
    // top-M select (no launch of their own between the two).
    const int nsl = dt::pers_slices(c.B), bsl = dt::pers_slice_b(c.B);
    bool fused = !marginal && !table && !noalloc && h->pp.ng > 0;
    bool pers = false;
    // (the cooperative launch only where asked for; otherwise a plain launch
    // of the same grid, whose co-residency rests on the occupancy check)
    const bool coop = c.expand == DT_EXPAND_PERSISTENT;
    const bool want_pers = c.expand == DT_EXPAND_PERSISTENT || c.expand == DT_EXPAND_RESIDENT;
    if (fused && (c.expand == DT_EXPAND_AUTO || want_pers)) {
        if (h->pers < 0) h->pers = dt::pers_supported(h->pp, bsl, c.V, c.E) ? 1 : 0;
        hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
        DT_TRY(hipStreamIsCapturing(st, &cs), "stream capture query");
        pers = h->pers == 1 && cs == hipStreamCaptureStatusNone;
        if (want_pers && !pers)
            return fail(h, DT_ERR_UNSUPPORTED, h->pers == 1
                                                   ? "persistent expansion: the stream is being captured"
                                                   : "persistent expansion: the device cannot hold the grid "
                                                     "(%d workgroups) at once, or V > 262143 or V E >= 2^31", h->pp.ng + bsl);
    }
    if (nsl > 1 && !pers) fused = false;  // (more requests than one launch step holds: stepped)
    dt::TopmSide side{};
    const int pslot = (int)h->calls.size() - 1;  // this call's clock pair, when timed
    unsigned long long* pclock = nullptr;
    if (pers) {
        side.zero = (unsigned*)(w + L.p_done) + h->pipe_T;  // from gflag on
        side.nzero = nsl * dt::pers_flag_words(h->pp, bsl);  // (every slice's)
        // (timed: the launch writes its device-clock span, which is the
        // stage's time; the events would span the cooperative launch's
        // hand-over as well)
        if (call && h->tlevel >= 2 && h->tclock && pslot < h->tclock_cap) pclock = h->tclock + 2 * (size_t)pslot;
        side.clock = pclock;
    }

    int32_t* tidx = (int32_t*)(w + L.tidx);
    float* tval = (float*)(w + L.tval);
    dt::LaunchEvents ev{};
    DT_TRY(kernel_marks(h, call, 1, 'K', 'T', &ev), "timing event");
    float* tail = c.full_vocab ? (float*)(w + L.tail) : nullptr;
    DT_TRY(dt::launch_topm(base, (int)c.dtype, c.B * c.L, c.V, h->nseg, (u64*)(w + L.partial), c.M,
                           tidx, tval, st, ev, tail_scale(c), tail, (float*)(w + L.tail_part), side),
           "top-M launch");
    if (h->nseg > 1) DT_TRY(mark(h, call, 1, 'M', st), "timing event");  // after the merge kernel

    dt::NodeArgs a{};
    a.B = c.B; a.L = c.L; a.V = c.V; a.E = c.E; a.H = c.H; a.M = c.M; a.n = c.n;
    a.dtype = (int)c.dtype;
    a.marginal = marginal ? 1 : 0;
    a.temp = c.temperature;
    a.eps = c.near_tie_eps;
    a.C = C; a.h0 = h0;
    a.tidx = tidx; a.tval = tval;
    a.b_ih = table ? nullptr : b_ih;  // folded into the table
    a.b_hh = b_hh;
    a.table = table;
    a.hstate = c.dtype == DT_F32 ? (float*)(w + L.hstate) : nullptr;
    a.hsplit = c.dtype == DT_BF16 ? (uint16_t*)(w + L.hsplit) : nullptr;
    a.partial = (const float*)(w + L.gpart);
    a.ksplit = table ? h->ksplit_f : h->ksplit;
    a.gru_tok = (int32_t*)(w + L.gru_tok);
    a.gru_par = (int32_t*)(w + L.gru_par);
    a.child_tok = (int32_t*)(w + L.child_tok);
    a.child_lp = (float*)(w + L.child_lp);
    a.ckey = (u64*)(w + L.ckey);
    a.queue = (u64*)(w + L.queue);
    a.rstate = (int32_t*)(w + L.rstate);
    a.nidx = (int32_t*)(w + L.nidx);
    a.nval = (float*)(w + L.nval);
    a.emb = emb;
    a.xpack = c.dtype == DT_BF16 && !marginal && !table ? (uint16_t*)(w + L.xpack) : nullptr;
    a.hpack = c.dtype == DT_BF16 && !marginal ? (uint16_t*)(w + L.hpack) : nullptr;
    a.hprev = c.dtype == DT_BF16 && !marginal ? (float*)(w + L.hprev) : nullptr;
    a.tail = tail;
    a.tokens = tokens; a.parents = parents; a.depths = depths; a.scores = scores;
    a.mask = mask; a.count = count; a.flags = flags;

    dt::GruGatesArgs g{};
    g.xpack = table ? a.hpack : a.xpack;  // (no x part when folded)
    g.hpack = a.hpack;
    g.x = emb;
    g.xtok = a.gru_tok;
    g.hf = a.hstate;
    g.hrows = c.n + 1;
    g.hsel = a.gru_par;
    g.W_ih = W_ih;
    g.W_hh = W_hh;
    g.partial = (float*)(w + L.gpart);
    g.B = c.B; g.E = table ? 0 : c.E; g.H = c.H;  // folded: the recurrent part alone
    g.ksplit = a.ksplit;
    g.dtype = (int)c.dtype;
    g.wpack = c.dtype == DT_BF16 && !noalloc ? (uint16_t*)(w + L.wpack) : nullptr;  // NULL: read in place

    if (marginal) {  // no contraction between the steps: one launch runs all n
        DT_TRY(kernel_marks(h, call, 2, 'n', 'N', &ev), "timing event");
        DT_TRY(dt::launch_marginal_build(a, h->lds, st, ev), "factorized expansion launch");
        DT_TRY(mark(h, call, 1, 'E', st), "timing event");
        return DT_OK;
    }
    if (fused) {  // fused expansion: n + 2 launches
        dt::PipeArgs pa{};
        pa.B = c.B; pa.L = c.L; pa.V = c.V; pa.E = c.E; pa.H = c.H; pa.M = c.M; pa.n = c.n;
        pa.T = h->pipe_T;
        pa.ng = h->pp.ng; pa.ksx = h->pp.ksx; pa.ksh = h->pp.ksh;
        pa.temp = c.temperature; pa.eps = c.near_tie_eps;
        pa.C = C; pa.h0 = h0; pa.tidx = tidx; pa.tval = tval; pa.tail = tail;
        pa.emb = emb; pa.W_ih = W_ih; pa.W_hh = W_hh; pa.b_ih = b_ih; pa.b_hh = b_hh;
        pa.xpack[0] = (uint16_t*)(w + L.xpack);
        pa.xpack[1] = (uint16_t*)(w + L.p_xpack1);
        pa.hpack[0] = (uint16_t*)(w + L.hpack);
        pa.hpack[1] = (uint16_t*)(w + L.p_hpack1);
        pa.xtok[0] = (int32_t*)(w + L.p_xtok);
        pa.xtok[1] = pa.xtok[0] + c.B;
        pa.hslot[0] = (int32_t*)(w + L.p_hslot);
        pa.hslot[1] = pa.hslot[0] + c.B;
        pa.gi = (float*)(w + L.p_gi);
        pa.gh = (float*)(w + L.p_gh);
        pa.hstate = (float*)(w + L.p_hstate);
        pa.exp_at = (int32_t*)(w + L.p_exp);
        pa.done = (unsigned*)(w + L.p_done);
        pa.gflag = pa.done + pa.T;
        pa.hflag = pa.gflag + pa.ng;
        pa.xflag = pa.hflag + 4 * pa.B;
        pa.perr = pa.xflag + 2 * pa.B;
        pa.active = (int32_t*)(w + L.p_active);
        pa.wpack = (uint16_t*)(w + L.wpack);
        pa.child_tok = a.child_tok; pa.child_lp = a.child_lp; pa.ckey = a.ckey; pa.queue = a.queue;
        pa.rstate = a.rstate; pa.nidx = a.nidx; pa.nval = a.nval;
        pa.tokens = tokens; pa.parents = parents; pa.depths = depths; pa.scores = scores;
        pa.mask = mask; pa.count = count; pa.flags = flags;
        h->last_mode = pers ? (coop ? DT_EXPAND_PERSISTENT : DT_EXPAND_RESIDENT) : DT_EXPAND_FUSED;
        if (pers) {
            DT_TRY(kernel_marks(h, call, 2, 'p', 'P', &ev), "timing event");
            if (pclock) {  // (set up before the top-M select)
                pa.tclock = pclock;
                call->back().clock = pslot;
            }
            // one launch per slice of requests, each on its own flag words;
            // the events (when timed) span them all
            const int S = c.n + 1, LM = c.L * c.M, H = c.H, fw = dt::pers_flag_words(h->pp, bsl);
            for (int sl = 0; sl < nsl; ++sl) {
                const int b0 = sl * bsl;
                const size_t r = (size_t)b0;
                dt::PipeArgs ps = pa;
                ps.B = std::min(bsl, c.B - b0);
                if (h0) ps.h0 = h0 + r * H;
                ps.tidx = tidx + r * LM;
                ps.tval = tval + r * LM;
                if (tail) ps.tail = tail + r * c.L;
                ps.gh = pa.gh + r * S * h->pp.ksh * 3 * H;
                ps.hstate = pa.hstate + r * S * H;
                ps.exp_at = pa.exp_at + r * S;
                ps.gflag = pa.gflag + (size_t)sl * fw;
                ps.hflag = ps.gflag + ps.ng;
                ps.xflag = ps.hflag + 4 * bsl;
                ps.perr = ps.xflag + 2 * bsl;
                ps.child_tok = pa.child_tok + r * S * 64;
                ps.child_lp = pa.child_lp + r * S * 64;
                ps.ckey = pa.ckey + r * S * 64;
                ps.queue = pa.queue + r * 64;
                ps.rstate = pa.rstate + r * dt::kStateWords;
                ps.nidx = pa.nidx + r * 64;
                ps.nval = pa.nval + r * 64;
                ps.tokens = tokens + r * S;
                ps.parents = parents + r * S;
                ps.depths = depths + r * S;
                ps.scores = scores + r * S;
                ps.mask = mask + r * S * S;
                ps.count = count + r;
                ps.flags = flags + r;
                dt::LaunchEvents es{sl == 0 ? ev.start : nullptr, sl == nsl - 1 ? ev.stop : nullptr};
                DT_TRY(dt::launch_pers_build(ps, h->pp, h->lds, st, es, coop), "persistent expansion launch");
            }
        } else {
            for (int t = 0; t < h->pipe_T; ++t) {
                DT_TRY(kernel_marks(h, call, 2, 'p', 'P', &ev), "timing event");
                DT_TRY(dt::launch_pipe_step(pa, h->pp, h->lds, t, st, ev), "fused expansion launch");
            }
        }
        DT_TRY(mark(h, call, 1, 'E', st), "timing event");
        return DT_OK;
    }
    if (!noalloc && !table) h->last_mode = DT_EXPAND_STEPPED;  // (a persistent plan that could not run)
    DT_TRY(kernel_marks(h, call, 2, 'n', 'N', &ev), "timing event");
    DT_TRY(dt::launch_node_step(a, h->lds, 0, st, ev), "node step launch");
    for (int step = 1; step < c.n; ++step) {
        // the first contraction of the call leaves the weights in operand
        // tiles; the later ones read that copy (contiguous 1 KB per wave load)
        g.wmode = c.dtype == DT_BF16 ? (step == 1 ? 1 : 2) : 0;
        DT_TRY(kernel_marks(h, call, 2, 'g', 'G', &ev), "timing event");
        DT_TRY(dt::launch_gru_gates(g, st, ev), "GRU contraction launch");
        DT_TRY(kernel_marks(h, call, 2, 'n', 'N', &ev), "timing event");
        DT_TRY(dt::launch_node_step(a, h->lds, step, st, ev), "node step launch");
    }
    DT_TRY(mark(h, call, 1, 'E', st), "timing event");
#undef DT_TRY
    return DT_OK;
}
}  // namespace

extern "C" {

dt_status dt_build(dt_handle* h, void* ws, size_t ws_bytes, const void* base, const void* emb,
                   const void* W_ih, const void* W_hh, const void* b_ih, const void* b_hh,
                   const void* C, const float* h0, int32_t* tokens, int32_t* parents, int32_t* depths,
                   float* scores, uint8_t* mask, int32_t* count, uint32_t* flags, void* stream) {
    return build_impl(false, h, ws, ws_bytes, base, emb, W_ih, W_hh, b_ih, b_hh, C, h0, tokens, parents,
                      depths, scores, mask, count, flags, stream);
}

dt_status dt_build_noalloc(dt_handle* h, const void* base, const void* emb, const void* W_ih, const void* W_hh,
                           const void* b_ih, const void* b_hh, const void* C, const float* h0, int32_t* tokens,
                           int32_t* parents, int32_t* depths, float* scores, uint8_t* mask, int32_t* count,
                           uint32_t* flags, void* stream) {
    return build_impl(false, h, nullptr, 0, base, emb, W_ih, W_hh, b_ih, b_hh, C, h0, tokens, parents, depths,
                      scores, mask, count, flags, stream, nullptr, /*noalloc=*/true);
}

dt_status dt_build_folded(dt_handle* h, void* ws, size_t ws_bytes, const void* base, const float* table,
                          const void* W_hh, const void* b_hh, const void* C, const float* h0, int32_t* tokens,
                          int32_t* parents, int32_t* depths, float* scores, uint8_t* mask, int32_t* count,
                          uint32_t* flags, void* stream) {
    if (h && !table) return fail(h, DT_ERR_INVALID_ARG, "dt_build_folded: null table");
    return build_impl(false, h, ws, ws_bytes, base, nullptr, nullptr, W_hh, nullptr, b_hh, C, h0, tokens, parents,
                      depths, scores, mask, count, flags, stream, table);
}

dt_status dt_fold_input(dt_handle* h, const void* emb, const void* W_ih, const void* b_ih, float* table,
                        void* stream) {
    if (!h) return DT_ERR_INVALID_ARG;
    const dt_config& c = h->cfg;
    if (!emb || !W_ih || !table) return fail(h, DT_ERR_INVALID_ARG, "dt_fold_input: null pointer");
    if (misaligned(emb) || misaligned(W_ih) || misaligned(b_ih) || misaligned(table))
        return fail(h, DT_ERR_INVALID_ARG, "dt_fold_input: buffers must be 16-byte aligned");
    if (dt_status s = pending_error(h)) return s;
    hipError_t e = dt::launch_fold(emb, W_ih, b_ih, table, c.V, c.E, c.H, (int)c.dtype, (hipStream_t)stream);
    return e == hipSuccess ? DT_OK : hip_fail(h, e, "dt_fold_input launch");
}

dt_status dt_build_marginal(dt_handle* h, void* ws, size_t ws_bytes, const void* base, int32_t* tokens,
                            int32_t* parents, int32_t* depths, float* scores, uint8_t* mask,
                            int32_t* count, uint32_t* flags, void* stream) {
    return build_impl(true, h, ws, ws_bytes, base, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr,
                      nullptr, tokens, parents, depths, scores, mask, count, flags, stream);
}

}  // extern "C"
