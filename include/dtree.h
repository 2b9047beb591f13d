/*
 * dtree.h -- C ABI of the MI355X (gfx950) conditional draft-tree builder.
 *
 * The library builds DominoTree's conditional best-first draft trees on the
 * GPU.  Sources, cited by site and section (arXiv:2607.08642, three pages):
 *   [captcha] "DominoTree: Conditional Tree-Structured Drafting with Domino for
 *             Speculative Decoding", blog.captcha.la research summary;
 *   [zhichai] zhichai.top post on the same paper;
 *   [gist]    gist.science explainer of the same paper (French).
 *
 * Conventions for every entry point below:
 *  - Pointers named as device buffers are device pointers (e.g. from
 *    torch.empty(..., device="cuda")).  They are BORROWED: the caller owns
 *    them and keeps them alive until the work enqueued on `stream` is done.
 *    Every matrix and table must be 16-byte aligned.
 *  - Layouts are row-major and dense.  "dtype" tensors have the handle's
 *    dt_config.dtype: IEEE binary32 (DT_F32) or bfloat16 (DT_BF16, stored as
 *    16-bit patterns).  Hidden states and all scores are binary32.
 *  - `stream` is a hipStream_t (NULL = the default stream).  Calls only
 *    enqueue work; none of them synchronizes.
 *  - Argument errors return DT_ERR_INVALID_ARG / DT_ERR_UNSUPPORTED /
 *    DT_ERR_WORKSPACE before anything is enqueued; dt_last_error() then holds
 *    a message.  A failed launch returns DT_ERR_HIP.  An error that earlier
 *    asynchronous HIP work left pending on the calling host thread (what
 *    hipGetLastError reports) is returned as DT_ERR_HIP, and cleared, by the
 *    next enqueueing call after its argument checks, before it enqueues
 *    anything.  Faults inside the kernels surface as HIP errors at the
 *    caller's next synchronization.
 *  - A handle is not thread-safe: one host thread at a time.  Overlapping
 *    calls that share a workspace race; give concurrent calls their own
 *    workspace.
 *  - Base logits must be finite (no NaN, no infinities).
 */
#ifndef DTREE_H
#define DTREE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    DT_OK = 0,
    DT_ERR_INVALID_ARG = -1, /* null pointer, bad size, misaligned buffer      */
    DT_ERR_UNSUPPORTED = -2, /* valid request outside what the library supports */
    DT_ERR_WORKSPACE = -3,   /* workspace missing or smaller than required     */
    DT_ERR_HIP = -4          /* a HIP runtime call or kernel launch failed      */
} dt_status;

typedef enum { DT_F32 = 0, DT_BF16 = 1 } dt_dtype;

/* Problem sizes, fixed at handle creation.
 *   B  requests per call (independent trees)          B >= 0
 *   L  block length = positions of base logits = max tree depth, 1..64
 *   V  vocabulary size                                 V >= 1, V < 2^31
 *   E  embedding width fed to the GRU                  bf16: multiple of 32; f32: multiple of 4
 *   H  GRU hidden width                                bf16: multiple of 32; f32: multiple of 4; <= 4096
 *   M  candidate width (top-M per position)            1..64, M <= V
 *   n  node budget: non-root nodes per tree            1..64
 *   temperature  0 = unscaled; > 0 divides the corrected logits before the
 *                log-softmax ([captcha] "Methodology -- deep read": runs at
 *                T in {0, 0.5, 1.0})
 *   near_tie_eps decisions closer than this are flagged (e.g. 1e-5)
 *   full_vocab   0: a node's children are normalized over its top-M slice;
 *                1: over the whole vocabulary, the corrected top-M logits
 *                plus the uncorrected logits of every other token of the
 *                row (the pages restrict the correction to the top M and
 *                leave the softmax scope open: [captcha] "Key findings",
 *                "Methodology -- deep read").  Applies to dt_build and
 *                dt_build_marginal.
 *   expand       how dt_build runs the expansion steps (same trees either
 *                way, up to binary32 rounding order of the GRU gate sums):
 *                DT_EXPAND_AUTO (0) resident (below) where the device and
 *                stream allow it and B <= 64, else fused where supported,
 *                else stepped; DT_EXPAND_STEPPED (1) two launches per step, the
 *                batched GRU contraction then the node step; DT_EXPAND_FUSED
 *                (2) one launch per step in which the contraction of the rows
 *                the requests need next runs beside the node steps (bf16,
 *                B <= 64, H <= 1024; otherwise dt_create returns
 *                DT_ERR_UNSUPPORTED); DT_EXPAND_PERSISTENT (3) the fused
 *                steps in one cooperative launch whose workgroups stay
 *                resident (the contraction keeps its weights in registers)
 *                and hand over through counters (bf16, H <= 1024; more than
 *                64 requests run as consecutive launches of 64 -- faster than
 *                stepped on shallow trees, slower on deep chains, where
 *                requests wait inside the steps; dt_build returns
 *                DT_ERR_UNSUPPORTED when the device cannot hold a launch's
 *                grid at once or the stream is being captured).  The same
 *                trees, bit for bit, as DT_EXPAND_FUSED, and for each slice
 *                of 64 requests as a call on those requests alone;
 *                DT_EXPAND_RESIDENT (4) the same kernel as a plain launch:
 *                the grid is resident by the occupancy check alone, not by
 *                the runtime's guarantee, and the call saves the cooperative
 *                launch's hand-over (about 20 us).  For a device the call
 *                does not share with long-running work: should another
 *                queue's kernels hold CUs for longer than the bounded waits
 *                (about 2^18 polls), the launch ends with flags bit 31 set
 *                for its requests rather than waiting longer.  The same
 *                trees, bit for bit, as DT_EXPAND_PERSISTENT.
 * A request's expansion state lives in one workgroup's LDS: configurations with
 * 4 H + 8 L M + 512 n bytes (plus ~0.8 KiB) above 64 KiB are DT_ERR_UNSUPPORTED. */
typedef enum {
    DT_EXPAND_AUTO = 0,
    DT_EXPAND_STEPPED = 1,
    DT_EXPAND_FUSED = 2,
    DT_EXPAND_PERSISTENT = 3,
    DT_EXPAND_RESIDENT = 4
} dt_expand;
typedef struct {
    int32_t B, L, V, E, H, M, n;
    float temperature;
    dt_dtype dtype;
    float near_tie_eps;
    int32_t full_vocab;
    int32_t expand;
} dt_config;

typedef struct dt_handle dt_handle; /* opaque: configuration, launch plan, timing events */

/* Validate `cfg` and create a handle.  Host only: no HIP call is made, so it
 * works without a GPU.  On error *out is NULL and the message is available
 * from dt_last_error(NULL). */
dt_status dt_create(const dt_config *cfg, dt_handle **out);
void dt_destroy(dt_handle *h);

/* Device workspace bytes dt_build needs for this handle (caller allocates,
 * 256-byte aligned).  dt_topm and dt_gru_step need no more than this. */
size_t dt_workspace_bytes(const dt_handle *h);

/* The expansion dt_build runs for this handle: DT_EXPAND_RESIDENT,
 * DT_EXPAND_PERSISTENT, DT_EXPAND_FUSED or DT_EXPAND_STEPPED -- the one its
 * last dt_build call ran, or before any call the one the configuration
 * selects (DT_EXPAND_AUTO with a fused plan: DT_EXPAND_RESIDENT, which a call
 * may turn into DT_EXPAND_FUSED, see dt_config.expand); -1 for a NULL handle.
 * Host only. */
int32_t dt_expand_mode(const dt_handle *h);

const char *dt_status_string(dt_status s);
/* Last error message of `h` (or of the last failed dt_create when h is NULL). */
const char *dt_last_error(const dt_handle *h);

/*
 * dt_build -- one speculative round's draft trees for B requests.
 *
 * The whole method runs on the device, with no host round trip:
 *  1. top-M marginal candidates per request and block position ([captcha]
 *     "Methodology -- deep read": per-node correction restricted to the
 *     marginal top-M tokens; [gist] "Composants clés -- Restriction de
 *     candidats (Top-M)");
 *  2. best-first expansion keyed by cumulative conditional log-prob until n
 *     nodes or the maximum depth L ([captcha] "Methodology -- deep read";
 *     [gist] "Composants clés -- Tas de recherche de premier choix à score
 *     conditionnel"); expanding node v advances the GRU hidden state by one
 *     step with v's token (gate order reset, update, new; both biases), then
 *     scores v's children over the top-M slice of block position depth(v):
 *     z_j = base[pos, idx_j] + C[idx_j] . h_v, z /= T when T > 0, log-softmax
 *     over the M-slice; children ranked by (log-prob desc, token id asc);
 *  3. the prefix-closed tree and its ancestor-only attention mask ([captcha]
 *     "Methodology -- deep read"; [gist] "Vérification").
 * Queue order: (score desc, depth asc, parent slot asc, sibling rank asc).
 * The hidden state is kept in binary32; in DT_BF16 the GRU's W_hh product
 * takes it as the exact sum of three bf16 parts (bf16 MFMA with binary32
 * accumulation), so the state is never rounded to bf16.
 *
 * Inputs (device, dtype unless noted):
 *   base_logits [B, L, V]   per-position base logits of each request
 *   emb         [V, E]      token embeddings (GRU input)
 *   W_ih [3H, E], W_hh [3H, H]; b_ih, b_hh [3H] or NULL (= zero)
 *   C           [V, H]      correction matrix
 *   h0          [B, H] binary32, or NULL (= zeros): hidden state at the root
 * Outputs (device; n+1 slots per request, slot 0 = root, slots in pop order):
 *   tokens  [B, n+1] int32   root -1; unused slots -1
 *   parents [B, n+1] int32   root -1; unused slots -1
 *   depths  [B, n+1] int32   root 0;  unused slots -1
 *   scores  [B, n+1] binary32 cumulative conditional log-prob; root 0; unused -inf
 *   mask    [B, n+1, n+1] uint8  mask[i][j] = 1 iff j == i or j is an ancestor
 *                                of i; rows of unused slots are 0
 *   count   [B] int32   non-root nodes built (< n only if the candidate tree
 *                       is smaller than n)
 *   flags   [B] uint32  bit 0: some pop beat a candidate left in the queue by
 *                       a positive binary32 margin below near_tie_eps (exact
 *                       ties are broken by the queue order, not flagged).
 *                       The popped node's next-ranked sibling is queued
 *                       before the comparison, so two children closer than
 *                       eps are such a pop, and the last pop's comparison
 *                       covers the final node set: every decision whose
 *                       outcome rounding could change sets this one bit.
 *                       Bit 31: (fused expansion) a wait for a launch's
 *                       contraction gave up after its bounded spin; the tree
 *                       is then not valid.  Other bits are 0.
 * workspace: device buffer of at least dt_workspace_bytes(h) bytes.
 */
dt_status dt_build(dt_handle *h, void *workspace, size_t ws_bytes, const void *base_logits,
                   const void *emb, const void *W_ih, const void *W_hh, const void *b_ih,
                   const void *b_hh, const void *C, const float *h0, int32_t *tokens,
                   int32_t *parents, int32_t *depths, float *scores, uint8_t *mask,
                   int32_t *count, uint32_t *flags, void *stream);

/*
 * dt_build_noalloc -- dt_build for callers that cannot allocate device
 * memory: code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc.  Same inputs, outputs and results as dt_build, bit for
 * bit; no workspace argument and no allocation of any kind: the scratch is a
 * static device array of the library, one per GPU (32 MiB), kept until the
 * process ends.  The weights are read in place (no operand-tile copy).
 *  - Configurations whose scratch need exceeds 32 MiB return
 *    DT_ERR_UNSUPPORTED before anything is enqueued (the Qwen3-4B and 8B
 *    shapes at B = 64 fit; the B = 256, n = 64 stress shape does not).
 *  - `stream` must belong to the calling thread's current device.
 *  - Every call on one GPU shares that GPU's scratch: calls that overlap on
 *    one GPU (other streams, other threads, other handles) race.  Calls
 *    ordered on one stream do not.  Nothing in the scratch needs clearing:
 *    each call writes what it reads.
 */
dt_status dt_build_noalloc(dt_handle *h, const void *base_logits, const void *emb, const void *W_ih,
                           const void *W_hh, const void *b_ih, const void *b_hh, const void *C,
                           const float *h0, int32_t *tokens, int32_t *parents, int32_t *depths,
                           float *scores, uint8_t *mask, int32_t *count, uint32_t *flags, void *stream);

/*
 * dt_build_marginal -- the same best-first builder with DDTree's factorized
 * scores: every node's children distribution is the log-softmax of the base
 * logits over the top-M slice of its block position (no GRU, no
 * correction), so a node's score is the sum of its tokens' marginal
 * log-probs ([zhichai] "DominoTree 的破局": DDTree's marginal scoring
 * function; [captcha] "Key findings": the marginal-scoring ablation).  The
 * result equals dt_build with C = 0.  Same handle, workspace, outputs,
 * temperature, tie orders and near-tie flags as dt_build; no GRU inputs.
 */
dt_status dt_build_marginal(dt_handle *h, void *workspace, size_t ws_bytes, const void *base_logits,
                            int32_t *tokens, int32_t *parents, int32_t *depths, float *scores,
                            uint8_t *mask, int32_t *count, uint32_t *flags, void *stream);

/*
 * dt_topm -- step 1 alone: per (request, position) row of base_logits
 * [B, L, V] (dtype), the M largest values ordered by (value desc, token id
 * asc).  Outputs idx [B, L, M] int32 and val [B, L, M] binary32 (exact input
 * values).  ([captcha] "Methodology -- deep read": the builder precomputes
 * the top-M marginal tokens per depth.)  Uses the workspace.
 */
dt_status dt_topm(dt_handle *h, void *workspace, size_t ws_bytes, const void *base_logits,
                  int32_t *idx, float *val, void *stream);

/*
 * dt_gru_step -- the GRU update alone, batched over B rows: h_out[b] =
 * GRUCell(x[b], h[b]) with x [B, E] (dtype), h [B, H] binary32, weights as in
 * dt_build, h_out [B, H] binary32.  ([captcha] "Methodology -- deep read": the
 * GRU hidden state is passed and updated along each candidate path.)  In
 * DT_BF16 the gate contraction runs on bf16 matrix cores with binary32
 * accumulation.  Uses the workspace.  h_out must not alias h.
 */
dt_status dt_gru_step(dt_handle *h, void *workspace, size_t ws_bytes, const void *x,
                      const float *h_in, const void *W_ih, const void *W_hh, const void *b_ih,
                      const void *b_hh, float *h_out, void *stream);

/*
 * dt_correct -- the conditional children distribution alone, one node per
 * request: with idx/val the top-M tables [B, L, M] (as from dt_topm), pos [B]
 * int32 the block position of each node's children (0..L-1), h [B, H]
 * binary32 the node's hidden state and C [V, H] (dtype): z_j = val[b, pos, j]
 * + C[idx[b, pos, j]] . h[b], z /= T when T > 0, log-softmax over the
 * M-slice, children ranked by (log-prob desc, token id asc) into
 * tok_sorted [B, M] int32 and logp_sorted [B, M] binary32.  ([captcha]
 * "Methodology -- deep read": rows of the correction matrices and base logits
 * of the top-M candidates are fetched; [gist] "Composants clés -- Restriction
 * de candidats (Top-M)".)  Needs no workspace.
 */
dt_status dt_correct(dt_handle *h, const int32_t *idx, const float *val, const void *C,
                     const float *h_in, const int32_t *pos, int32_t *tok_sorted,
                     float *logp_sorted, void *stream);

/*
 * Folded input projection.  A node's GRU input is the embedding of its own
 * token ([captcha] "Methodology -- deep read": the GRU state is advanced
 * with the realized tokens of the path), so b_ih + W_ih . x takes one of V
 * values, fixed by the model.
 *
 * dt_fold_input computes them once: table [V, 3H] binary32 (caller-owned,
 * 16-byte aligned; 3 * 4 * H * V bytes, 1.9 GB at V = 151936, H = 1024),
 * table[v][g H + u] = b_ih[g H + u] + sum_k W_ih[g H + u][k] * emb[v][k]
 * (gate order r, z, n; b_ih may be NULL).  emb [V, E] and W_ih [3H, E] in
 * the handle's dtype.  fp32 accumulation (bf16 products are exact).
 *
 * dt_build_folded is dt_build with that table in place of emb, W_ih and
 * b_ih: each step's gate contraction covers the recurrent part W_hh . h
 * alone and the node step adds the popped token's table row.  Same outputs
 * as dt_build up to binary32 rounding order.  Errors as dt_build (a NULL
 * table is DT_ERR_INVALID_ARG).
 */
dt_status dt_fold_input(dt_handle *h, const void *emb, const void *W_ih, const void *b_ih, float *table,
                        void *stream);
dt_status dt_build_folded(dt_handle *h, void *workspace, size_t ws_bytes, const void *base,
                          const float *table, const void *W_hh, const void *b_hh, const void *C,
                          const float *h0, int32_t *tokens, int32_t *parents, int32_t *depths,
                          float *scores, uint8_t *mask, int32_t *count, uint32_t *flags, void *stream);

/*
 * dt_topm_tail -- dt_topm plus each row's tail mass: tail[b][p] = log of the
 * sum of exp(x / T) (T = 1 when temperature = 0) over the logits x of row
 * (b, p) outside its top M; -inf when M = V.  This is the extra term of the
 * full-vocabulary normalizer (see dt_config.full_vocab), computed in the
 * same single pass over the logits: every element outside the final top M
 * is added exactly once.
 *   base [B, L, V] dtype; idx [B, L, M] int32, val [B, L, M] binary32,
 *   tail [B, L] binary32 (out).  Workspace as for dt_build.
 * Errors as dt_topm.
 */
dt_status dt_topm_tail(dt_handle *h, void *workspace, size_t ws_bytes, const void *base, int32_t *idx,
                       float *val, float *tail, void *stream);

/*
 * dt_accept_greedy -- greedy (temperature 0) acceptance of B verified trees.
 *
 * After one target forward pass over the tree (ancestor-only mask), serial
 * greedy decoding agrees with the draft along one root path: at the current
 * node, first the root, the target's greedy token selects the child carrying
 * it, and the walk stops at a node with no such child; the target's token
 * there is also emitted, so a round yields accepted + 1 tokens
 * ([captcha] "Methodology -- deep read": the longest accepted root-to-leaf
 * path of one verification pass; [gist] "Résultats expérimentaux -- Absence
 * de perte": lossless against serial greedy decoding).
 *
 *   tokens, parents [B, n+1] int32, count [B] int32: a tree as dt_build
 *                   writes it (slot 0 = root; slots 1..count are nodes;
 *                   count is clamped to [0, n]).  Children of one node
 *                   should carry distinct tokens; if two match, the lower
 *                   slot is taken.
 *   target [B, n+1] int32: target[b][i] = the target model's greedy token
 *                   after the prefix that ends at node i (slot 0: after the
 *                   context); slots past count are not read.
 *   path   [B, n+1] int32 (out): the accepted slots in order, then -1.
 *   accepted [B] int32 (out): number of accepted draft tokens (0..n).
 *   bonus    [B] int32 (out): the target's token at the last accepted node.
 *
 * Device pointers, borrowed; asynchronous on `stream`; B = 0 is a no-op.
 * Errors: DT_ERR_INVALID_ARG for a null pointer (before any launch),
 * DT_ERR_HIP if the launch fails.  Uses no workspace.
 */
dt_status dt_accept_greedy(dt_handle *h, const int32_t *tokens, const int32_t *parents,
                           const int32_t *count, const int32_t *target, int32_t *path,
                           int32_t *accepted, int32_t *bonus, void *stream);

/*
 * Stage timing for benchmarks.  dt_timing_enable(h, level, capacity) makes
 * the next `capacity` dt_build (or dt_accept_greedy) calls record HIP events
 * on their stream:
 * level 1 on the top-M select kernel only, level 2 on every kernel; level 0
 * turns timing off and drops recorded events.  A kernel's events are taken
 * by its launch (hipExtLaunchKernel), so they span the kernel alone, not the
 * dispatch gap before it.  After the stream is synchronized,
 * dt_timing_read(h, stage, ms, max, n_out) returns per-call durations in
 * milliseconds, oldest first:
 *   stage 0  top-M select kernel (one launch per call)
 *   stage 1  top-M merge kernel, with the gap before it (no entries when
 *            each row is one segment and no merge kernel runs)
 *   stage 2  GRU gate contractions of the call, summed   (level 2)
 *   stage 3  node (correction + queue) kernels, summed    (level 2)
 *   stage 4  the whole call
 *   stage 5  GRU gate contraction, every launch separately (level 2)
 *   stage 6  the dt_accept_greedy kernel (one launch per call)
 *   stage 7  fused expansion launches of the call, summed  (level 2)
 *   stage 8  fused expansion, every launch separately      (level 2; the
 *            persistent expansion is one launch per call, timed by the
 *            device's constant 100 MHz clock from its first workgroup's
 *            start to its last one's end: events around a cooperative
 *            launch would also span its hand-over between queues)
 * Timing calls are host-side and need the handle's device to be current.
 */
dt_status dt_timing_enable(dt_handle *h, int level, int capacity);
dt_status dt_timing_read(dt_handle *h, int stage, float *ms, int max, int *n_out);

#ifdef __cplusplus
}
#endif

#endif /* DTREE_H */
