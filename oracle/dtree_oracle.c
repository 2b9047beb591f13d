/*
 * dtree_oracle.c -- CPU oracle for DominoTree's conditional best-first
 * draft-tree builder.
 *
 * TEST INFRASTRUCTURE ONLY.  This file is the plain, slow, single-threaded
 * reference that the GPU library is checked against.  Only the test suite,
 * the smoke check and the CPU-baseline leg of the benchmark may load it.  It
 * shares no code, header, table or helper with the GPU library.
 *
 * Sources (the three web pages on arXiv:2607.08642, cited by site and
 * section):
 *   [captcha]  "DominoTree: Conditional Tree-Structured Drafting with Domino
 *              for Speculative Decoding", blog.captcha.la research summary.
 *   [zhichai]  "DominoTree：让推测解码的多米诺骨牌自己长出一棵树",
 *              zhichai.top post.
 *   [gist]     gist.science explainer of the same paper (French).
 *
 * What it computes, per request:
 *   1. the top-M marginal candidates of every block position
 *      ([captcha] "Methodology -- deep read": the per-node correction is
 *      restricted to the marginal top-M tokens, whose correction-matrix rows
 *      and base logits are fetched; the builder "precomputes top-M marginal
 *      tokens per depth"; [gist] "Composants clés -- Restriction de
 *      candidats (Top-M)");
 *   2. for every expanded node, the GRU hidden state advanced by one step
 *      with the node's realized token ([captcha] "Methodology -- deep read":
 *      the GRU hidden state is passed and updated along each candidate path;
 *      [gist] "Composants clés": only the light GRU correction and the
 *      correction head are recomputed per node);
 *   3. the node's children distribution: base logit plus the correction
 *      (gathered correction-matrix row times the hidden state), over the
 *      M-slice, then a log-softmax over that slice;
 *   4. DDTree's best-first expansion with a max-priority queue keyed by the
 *      cumulative conditional log-probability, until the node budget n or
 *      the maximum depth ([captcha] "Methodology -- deep read"; [gist]
 *      "Composants clés -- Tas de recherche de premier choix à score
 *      conditionnel");
 *   5. the prefix-closed tree and its ancestor-only attention mask
 *      ([captcha] "Methodology -- deep read"; [gist] "Vérification");
 *   6. after verification at temperature 0, the accepted path: the target's
 *      greedy token at each node decides which child, if any, is accepted
 *      next ([captcha] "Methodology -- deep read": the longest accepted
 *      root-to-leaf path of one target forward pass; [gist] "Résultats
 *      expérimentaux -- Absence de perte": the output equals serial greedy
 *      decoding).
 *
 * Readings of points the pages leave open:
 *   - nodes at depth d take their tokens from block position d-1, so the
 *     maximum depth equals the block length L;
 *   - the GRU is the textbook cell with gate order (reset, update, new) and
 *     both bias vectors; the correction is C[token] . h with no bias;
 *   - the log-softmax runs over the M-slice only; a temperature T > 0
 *     divides the corrected logits first, T = 0 means unscaled;
 *   - the budget n counts non-root nodes; children are pushed lazily (the
 *     next-ranked sibling enters the queue when its elder sibling is
 *     popped), which yields the same n best nodes as pushing all children;
 *   - ties: children are ranked by (log-prob desc, token id asc); queue
 *     entries by (score desc, depth asc, parent pop index asc, sibling rank
 *     asc), a total order;
 *   - near ties: at each pop, every candidate left in the queue whose score
 *     is within eps of the popped one is a near tie, unless both scores are
 *     sums of the identical sequence of log-prob terms (exact zeros
 *     dropped), which every floating-point evaluation ties exactly; the
 *     smallest gap to a candidate not tied that way (0 included) is reported,
 *     and a flag is raised when it is below eps.  Losslessness only holds up to floating-point
 *     tie-breaking ([captcha] "Threat model"; [gist] "Résultats
 *     expérimentaux -- Absence de perte"): mathematically equal scores
 *     reached through different additions are such tie-breaks;
 *   - the hidden state is a real-valued state: it is never rounded to the
 *     storage type of the weights (the pages fix no precision for it);
 *   - full-vocabulary normalization (an optional mode): the pages say the
 *     per-node correction is restricted to the top-M candidates and that
 *     the restriction leaves the tree shape unchanged ([captcha] "Key
 *     findings", "Methodology -- deep read"), but not over which tokens the
 *     softmax runs.  In this mode a node's children are normalized over the
 *     whole vocabulary: the corrected top-M logits plus the uncorrected
 *     logits of every other token (the tail), i.e. the normalizer adds
 *     exp(tail_lse) with tail_lse = log sum over v outside the top-M of
 *     exp(base_v / T) (T = 1 when T = 0).  The default mode normalizes over
 *     the M-slice only.
 *
 * Arithmetic is double precision throughout; fp32 and bf16 inputs are
 * widened exactly.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define OR_F32 0
#define OR_BF16 1

#define OR_OK 0
#define OR_EINVAL (-1)
#define OR_ENOMEM (-2)

/* ---- exact widening of the stored inputs --------------------------------- */

static double load_elem(const void *p, int dtype, size_t i)
{
    if (dtype == OR_F32)
        return (double)((const float *)p)[i];
    /* a bf16 value is the upper half of an IEEE binary32 value */
    uint32_t bits = (uint32_t)((const uint16_t *)p)[i] << 16;
    float f;
    memcpy(&f, &bits, sizeof f);
    return (double)f;
}

/* ---- 1. top-M marginal candidates of one block position ------------------ */

typedef struct {
    double v;
    int32_t id;
} cand_t;

/* value descending, then token id ascending: a total order */
static int cand_cmp(const void *a, const void *b)
{
    const cand_t *x = (const cand_t *)a, *y = (const cand_t *)b;
    if (x->v > y->v) return -1;
    if (x->v < y->v) return 1;
    return (x->id > y->id) - (x->id < y->id);
}

int oracle_topm_row(const void *row, int dtype, int V, int M, int32_t *idx, double *val)
{
    if (!row || !idx || !val || V < 1 || M < 1 || M > V) return OR_EINVAL;
    cand_t *c = (cand_t *)malloc((size_t)V * sizeof *c);
    if (!c) return OR_ENOMEM;
    for (int t = 0; t < V; ++t) {
        c[t].v = load_elem(row, dtype, (size_t)t);
        c[t].id = t;
    }
    qsort(c, (size_t)V, sizeof *c, cand_cmp);
    for (int j = 0; j < M; ++j) {
        idx[j] = c[j].id;
        val[j] = c[j].v;
    }
    free(c);
    return OR_OK;
}

/* Log of the summed exponentials of the row's logits outside its top-M set
 * idx[0..M), each divided by T when T > 0 (full-vocabulary normalization);
 * -inf when the top-M set is the whole row. */
int oracle_tail_lse(const void *row, int dtype, int V, int M, double T, const int32_t *idx, double *out)
{
    if (!row || !idx || !out || V < 1 || M < 1 || M > V || T < 0.0) return OR_EINVAL;
    unsigned char *in_top = (unsigned char *)calloc((size_t)V, 1);
    if (!in_top) return OR_ENOMEM;
    for (int j = 0; j < M; ++j) {
        if (idx[j] < 0 || idx[j] >= V) { free(in_top); return OR_EINVAL; }
        in_top[idx[j]] = 1;
    }
    const double scale = T > 0.0 ? 1.0 / T : 1.0;
    double mx = -INFINITY;
    for (int t = 0; t < V; ++t)
        if (!in_top[t]) {
            double x = load_elem(row, dtype, (size_t)t) * scale;
            if (x > mx) mx = x;
        }
    double sum = 0.0;
    if (mx > -INFINITY)
        for (int t = 0; t < V; ++t)
            if (!in_top[t]) sum += exp(load_elem(row, dtype, (size_t)t) * scale - mx);
    *out = sum > 0.0 ? mx + log(sum) : -INFINITY;
    free(in_top);
    return OR_OK;
}

/* ---- 2. one GRU step ------------------------------------------------------ */

static double sigm(double x) { return 1.0 / (1.0 + exp(-x)); }

/* h_out = GRUCell(x, h): rows [0,H) of the weights are the reset gate,
 * [H,2H) the update gate, [2H,3H) the new-state gate.  x is row `xrow` of
 * the embedding-like matrix `xmat` ([*, E]).  Biases may be NULL (zero). */
int oracle_gru(const void *xmat, int64_t xrow, int dtype, const double *h,
               const void *W_ih, const void *W_hh, const void *b_ih, const void *b_hh,
               int E, int H, double *h_out)
{
    if (!xmat || !h || !W_ih || !W_hh || !h_out || E < 1 || H < 1 || xrow < 0)
        return OR_EINVAL;
    double *x = (double *)malloc((size_t)E * sizeof *x);
    if (!x) return OR_ENOMEM;
    for (int k = 0; k < E; ++k)
        x[k] = load_elem(xmat, dtype, (size_t)xrow * (size_t)E + (size_t)k);

    for (int o = 0; o < H; ++o) {
        double gi[3], gh[3];
        for (int g = 0; g < 3; ++g) {
            size_t row = (size_t)g * (size_t)H + (size_t)o;
            double si = b_ih ? load_elem(b_ih, dtype, row) : 0.0;
            for (int k = 0; k < E; ++k)
                si += load_elem(W_ih, dtype, row * (size_t)E + (size_t)k) * x[k];
            double sh = b_hh ? load_elem(b_hh, dtype, row) : 0.0;
            for (int k = 0; k < H; ++k)
                sh += load_elem(W_hh, dtype, row * (size_t)H + (size_t)k) * h[k];
            gi[g] = si;
            gh[g] = sh;
        }
        double r = sigm(gi[0] + gh[0]);
        double u = sigm(gi[1] + gh[1]);
        double c = tanh(gi[2] + r * gh[2]);
        h_out[o] = (1.0 - u) * c + u * h[o];
    }
    free(x);
    return OR_OK;
}

/* ---- 3. corrected, normalized children distribution ---------------------- */

typedef struct {
    double lp;
    int32_t tok;
} child_t;

/* log-prob descending, then token id ascending */
static int child_cmp(const void *a, const void *b)
{
    const child_t *x = (const child_t *)a, *y = (const child_t *)b;
    if (x->lp > y->lp) return -1;
    if (x->lp < y->lp) return 1;
    return (x->tok > y->tok) - (x->tok < y->tok);
}

/* z_j = val_j + C[idx_j] . h ; z /= T if T > 0 ; log-softmax over j < M,
 * with exp(tail) added to the normalizer (tail = -inf: the M-slice alone;
 * else the full-vocabulary mode's tail_lse of the node's row) ; children
 * sorted by (log-prob desc, token asc). */
int oracle_dist(const int32_t *idx, const double *val, int M, const void *C, int dtype,
                int H, const double *h, double T, double tail, int32_t *tok_sorted, double *lp_sorted)
{
    if (!idx || !val || !C || !h || !tok_sorted || !lp_sorted || M < 1 || H < 1 || T < 0.0)
        return OR_EINVAL;
    double *z = (double *)malloc((size_t)M * sizeof *z);
    child_t *ch = (child_t *)malloc((size_t)M * sizeof *ch);
    if (!z || !ch) { free(z); free(ch); return OR_ENOMEM; }
    for (int j = 0; j < M; ++j) {
        double d = 0.0;
        size_t base = (size_t)idx[j] * (size_t)H;
        for (int k = 0; k < H; ++k)
            d += load_elem(C, dtype, base + (size_t)k) * h[k];
        z[j] = val[j] + d;
        if (T > 0.0) z[j] = z[j] / T;
    }
    double m = z[0];
    for (int j = 1; j < M; ++j)
        if (z[j] > m) m = z[j];
    if (tail > m) m = tail;
    double s = 0.0;
    for (int j = 0; j < M; ++j)
        s += exp(z[j] - m);
    if (tail > -INFINITY) s += exp(tail - m);
    double ls = log(s);
    for (int j = 0; j < M; ++j) {
        ch[j].lp = (z[j] - m) - ls;
        ch[j].tok = idx[j];
    }
    qsort(ch, (size_t)M, sizeof *ch, child_cmp);
    for (int j = 0; j < M; ++j) {
        tok_sorted[j] = ch[j].tok;
        lp_sorted[j] = ch[j].lp;
    }
    free(z);
    free(ch);
    return OR_OK;
}

/* ---- 4. best-first expansion with a max-priority queue ------------------- */

typedef struct {
    double score; /* cumulative conditional log-prob of the candidate node */
    int depth;    /* depth the candidate would take */
    int parent;   /* pop index (tree slot) of its parent */
    int rank;     /* its rank among the parent's sorted children */
} qent_t;

/* Log-prob terms along the path of a candidate (parent q, rank r): the
 * parent's path terms, then the candidate's own log-prob; exact zeros are
 * dropped because adding 0 never changes a floating-point sum. */
static int path_terms(const double *plp, const int *plen, const double *clp, int L, int M,
                      const qent_t *c, double *out)
{
    int k = 0;
    for (int i = 0; i < plen[c->parent]; ++i) {
        double t = plp[(size_t)c->parent * L + i];
        if (t != 0.0) out[k++] = t;
    }
    double t = clp[(size_t)c->parent * M + c->rank];
    if (t != 0.0) out[k++] = t;
    return k;
}

/* 1 when the two candidates' scores add the identical sequence of terms */
static int same_terms(const double *plp, const int *plen, const double *clp, int L, int M,
                      const qent_t *a, const qent_t *b, double *wa, double *wb)
{
    int na = path_terms(plp, plen, clp, L, M, a, wa);
    int nb = path_terms(plp, plen, clp, L, M, b, wb);
    if (na != nb) return 0;
    for (int i = 0; i < na; ++i)
        if (wa[i] != wb[i]) return 0;
    return 1;
}

/* 1 when a comes before b in the queue's total order */
static int q_before(const qent_t *a, const qent_t *b)
{
    if (a->score != b->score) return a->score > b->score;
    if (a->depth != b->depth) return a->depth < b->depth;
    if (a->parent != b->parent) return a->parent < b->parent;
    return a->rank < b->rank;
}

typedef struct {
    qent_t *e;
    int size;
} queue_t;

static void q_push(queue_t *q, qent_t x)
{
    int i = q->size++;
    q->e[i] = x;
    while (i > 0) {
        int p = (i - 1) / 2;
        if (!q_before(&q->e[i], &q->e[p])) break;
        qent_t t = q->e[i]; q->e[i] = q->e[p]; q->e[p] = t;
        i = p;
    }
}

static qent_t q_pop(queue_t *q)
{
    qent_t top = q->e[0];
    q->e[0] = q->e[--q->size];
    int i = 0;
    for (;;) {
        int l = 2 * i + 1, r = l + 1, best = i;
        if (l < q->size && q_before(&q->e[l], &q->e[best])) best = l;
        if (r < q->size && q_before(&q->e[r], &q->e[best])) best = r;
        if (best == i) break;
        qent_t t = q->e[i]; q->e[i] = q->e[best]; q->e[best] = t;
        i = best;
    }
    return top;
}

/*
 * Build the tree of one request.
 *
 * Inputs (dtype-typed unless noted; row-major):
 *   base [L,V]  the block's per-position base logits (this request only)
 *   emb  [V,E]  token embeddings fed to the GRU
 *   W_ih [3H,E], W_hh [3H,H], b_ih [3H] | NULL, b_hh [3H] | NULL
 *   C    [V,H]  correction matrix
 *   h0   [H]    fp32 initial hidden state, or NULL for zeros
 *   T           temperature (0 = unscaled)
 *   eps         near-tie threshold
 * Outputs (n+1 tree slots; slot 0 is the root):
 *   tokens/parents/depths [n+1] int32, scores [n+1] double, mask [(n+1)^2],
 *   count (non-root nodes built), flags (bit 0: a near tie below eps),
 *   min_gap (smallest gap between a popped candidate and one left in the
 *   queue, structural exact ties excluded; +inf if the queue was always empty),
 *   first_flag (optional, may be NULL): the slot created by the first pop
 *   whose gap to a candidate left in the queue was below eps (0 when no pop
 *   was), so slots 1 .. first_flag-1 were decided by margins of at least eps,
 *   topm_idx/topm_val [L,M] (optional, may be NULL);
 *   full_vocab  0: children normalized over the M-slice; 1: over the whole
 *               vocabulary (corrected top-M plus the uncorrected tail);
 *   tail_out [L] (optional): the per-position tail_lse (-inf in the
 *               M-slice mode).
 */
int oracle_build_request(int V, int L, int E, int H, int M, int n, double T, int dtype, double eps,
                         const void *base, const void *emb, const void *W_ih, const void *W_hh,
                         const void *b_ih, const void *b_hh, const void *C, const float *h0,
                         int32_t *tokens, int32_t *parents, int32_t *depths, double *scores,
                         uint8_t *mask, int32_t *count, uint32_t *flags, double *min_gap,
                         int32_t *topm_idx, double *topm_val, int full_vocab, double *tail_out,
                         int32_t *first_flag)
{
    if (V < 1 || L < 1 || E < 1 || H < 1 || M < 1 || M > V || n < 1 || T < 0.0 ||
        (dtype != OR_F32 && dtype != OR_BF16) || !base || !emb || !W_ih || !W_hh || !C ||
        !tokens || !parents || !depths || !scores || !mask || !count || !flags || !min_gap)
        return OR_EINVAL;

    const int S = n + 1; /* tree slots */
    int rc = OR_ENOMEM;
    int32_t *tidx = (int32_t *)malloc((size_t)L * M * sizeof *tidx);
    double *tval = (double *)malloc((size_t)L * M * sizeof *tval);
    double *hs = (double *)malloc((size_t)S * H * sizeof *hs);
    int32_t *ctok = (int32_t *)malloc((size_t)S * M * sizeof *ctok);
    double *clp = (double *)malloc((size_t)S * M * sizeof *clp);
    double *plp = (double *)malloc((size_t)S * L * sizeof *plp); /* path terms per slot */
    int *plen = (int *)malloc((size_t)S * sizeof *plen);
    double *wa = (double *)malloc((size_t)(L + 1) * sizeof *wa);
    double *wb = (double *)malloc((size_t)(L + 1) * sizeof *wb);
    double *tail = (double *)malloc((size_t)L * sizeof *tail);
    queue_t q = {(qent_t *)malloc((size_t)(2 * S + 2) * sizeof(qent_t)), 0};
    if (!tidx || !tval || !hs || !ctok || !clp || !plp || !plen || !wa || !wb || !tail || !q.e) goto done;

    /* 1. top-M marginal candidates per block position */
    const size_t esz = (dtype == OR_F32) ? 4 : 2;
    for (int p = 0; p < L; ++p) {
        const char *row = (const char *)base + (size_t)p * (size_t)V * esz;
        rc = oracle_topm_row(row, dtype, V, M, tidx + (size_t)p * M, tval + (size_t)p * M);
        if (rc) goto done;
        tail[p] = -INFINITY;
        if (full_vocab) {
            rc = oracle_tail_lse(row, dtype, V, M, T, tidx + (size_t)p * M, tail + p);
            if (rc) goto done;
        }
    }

    /* empty tree */
    for (int i = 0; i < S; ++i) {
        tokens[i] = -1; parents[i] = -1; depths[i] = -1; scores[i] = -INFINITY;
    }
    memset(mask, 0, (size_t)S * S);
    *flags = 0;
    *min_gap = INFINITY;
    int first = 0;

    /* root: slot 0, depth 0, score 0, hidden state h0; its children sit at
     * depth 1 and take their tokens from block position 0 */
    depths[0] = 0;
    scores[0] = 0.0;
    plen[0] = 0;
    for (int k = 0; k < H; ++k) hs[k] = h0 ? (double)h0[k] : 0.0;
    rc = oracle_dist(tidx, tval, M, C, dtype, H, hs, T, tail[0], ctok, clp);
    if (rc) goto done;
    q_push(&q, (qent_t){0.0 + clp[0], 1, 0, 0});

    int built = 0;
    while (built < n && q.size > 0) {
        qent_t c = q_pop(&q);
        int v = ++built;
        tokens[v] = ctok[(size_t)c.parent * M + c.rank];
        parents[v] = c.parent;
        depths[v] = c.depth;
        scores[v] = c.score;
        plen[v] = plen[c.parent] + 1;
        for (int i = 0; i < plen[c.parent]; ++i)
            plp[(size_t)v * L + i] = plp[(size_t)c.parent * L + i];
        plp[(size_t)v * L + plen[c.parent]] = clp[(size_t)c.parent * M + c.rank];
        /* the popped node's next-ranked sibling becomes a candidate */
        if (c.rank + 1 < M)
            q_push(&q, (qent_t){scores[c.parent] + clp[(size_t)c.parent * M + c.rank + 1], c.depth,
                                c.parent, c.rank + 1});
        /* near-tie bookkeeping: gaps to the candidates left in the queue */
        for (int i = 0; i < q.size; ++i) {
            double gap = c.score - q.e[i].score;
            if (gap >= *min_gap) continue;
            if (gap == 0.0 && same_terms(plp, plen, clp, L, M, &c, &q.e[i], wa, wb)) continue;
            *min_gap = gap;
            if (!first && gap < eps) first = v;
        }
        /* expand: GRU step with the realized token, then score its children
         * at block position depth(v).  Nodes at the maximum depth have no
         * children; the last node's children could never be popped. */
        if (c.depth < L && built < n) {
            double *hv = hs + (size_t)v * H;
            rc = oracle_gru(emb, tokens[v], dtype, hs + (size_t)c.parent * H, W_ih, W_hh, b_ih, b_hh,
                            E, H, hv);
            if (rc) goto done;
            rc = oracle_dist(tidx + (size_t)c.depth * M, tval + (size_t)c.depth * M, M, C, dtype, H,
                             hv, T, tail[c.depth], ctok + (size_t)v * M, clp + (size_t)v * M);
            if (rc) goto done;
            q_push(&q, (qent_t){scores[v] + clp[(size_t)v * M], c.depth + 1, v, 0});
        }
    }
    *count = built;
    if (*min_gap < eps) *flags |= 1u;
    if (first_flag) *first_flag = first;

    /* 5. ancestor-only mask: row i attends to itself and its ancestors */
    for (int i = 0; i <= built; ++i)
        for (int j = i; j >= 0; j = parents[j])
            mask[(size_t)i * S + j] = 1;

    if (topm_idx) memcpy(topm_idx, tidx, (size_t)L * M * sizeof *tidx);
    if (topm_val) memcpy(topm_val, tval, (size_t)L * M * sizeof *tval);
    if (tail_out) memcpy(tail_out, tail, (size_t)L * sizeof *tail);
    rc = OR_OK;
done:
    free(tidx); free(tval); free(hs); free(ctok); free(clp); free(plp); free(plen); free(wa);
    free(wb); free(tail); free(q.e);
    return rc;
}

/*
 * Conditional score of arbitrary token paths of one request (used to check
 * a tree whose order was decided by a near tie): for path i, given as tokens
 * paths[i*L .. i*L+len[i]), returns the cumulative conditional log-prob of
 * its last node, or -inf when a token is not among its depth's top-M.
 */
int oracle_score_paths(int V, int L, int E, int H, int M, double T, int dtype, const void *base,
                       const void *emb, const void *W_ih, const void *W_hh, const void *b_ih,
                       const void *b_hh, const void *C, const float *h0, int npaths,
                       const int32_t *paths, const int32_t *len, double *out, int full_vocab)
{
    if (V < 1 || L < 1 || E < 1 || H < 1 || M < 1 || M > V || npaths < 0 || T < 0.0 || !base ||
        !emb || !W_ih || !W_hh || !C || (npaths > 0 && (!paths || !len || !out)))
        return OR_EINVAL;
    int rc = OR_ENOMEM;
    int32_t *tidx = (int32_t *)malloc((size_t)L * M * sizeof *tidx);
    double *tval = (double *)malloc((size_t)L * M * sizeof *tval);
    double *h = (double *)malloc((size_t)H * sizeof *h);
    double *h2 = (double *)malloc((size_t)H * sizeof *h2);
    int32_t *ctok = (int32_t *)malloc((size_t)M * sizeof *ctok);
    double *clp = (double *)malloc((size_t)M * sizeof *clp);
    double *tail = (double *)malloc((size_t)L * sizeof *tail);
    if (!tidx || !tval || !h || !h2 || !ctok || !clp || !tail) goto done;
    const size_t esz = (dtype == OR_F32) ? 4 : 2;
    for (int p = 0; p < L; ++p) {
        const char *row = (const char *)base + (size_t)p * V * esz;
        rc = oracle_topm_row(row, dtype, V, M, tidx + (size_t)p * M, tval + (size_t)p * M);
        if (rc) goto done;
        tail[p] = -INFINITY;
        if (full_vocab) {
            rc = oracle_tail_lse(row, dtype, V, M, T, tidx + (size_t)p * M, tail + p);
            if (rc) goto done;
        }
    }
    for (int i = 0; i < npaths; ++i) {
        int d = len[i];
        if (d < 1 || d > L) { rc = OR_EINVAL; goto done; }
        for (int k = 0; k < H; ++k) h[k] = h0 ? (double)h0[k] : 0.0;
        double s = 0.0;
        for (int p = 0; p < d; ++p) {
            int32_t tok = paths[(size_t)i * L + p];
            rc = oracle_dist(tidx + (size_t)p * M, tval + (size_t)p * M, M, C, dtype, H, h, T, tail[p], ctok,
                             clp);
            if (rc) goto done;
            int r = -1;
            for (int j = 0; j < M; ++j)
                if (ctok[j] == tok) { r = j; break; }
            if (r < 0) { s = -INFINITY; break; }
            s += clp[r];
            if (p + 1 < d) {
                rc = oracle_gru(emb, tok, dtype, h, W_ih, W_hh, b_ih, b_hh, E, H, h2);
                if (rc) goto done;
                memcpy(h, h2, (size_t)H * sizeof *h);
            }
        }
        out[i] = s;
    }
    rc = OR_OK;
done:
    free(tidx); free(tval); free(h); free(h2); free(ctok); free(clp); free(tail);
    return rc;
}

/*
 * Greedy (temperature 0) acceptance of one request's verified tree.
 *
 * The tree is the builder's output: slots 0..count, slot 0 the root,
 * tokens[i] and parents[i] for i >= 1.  target[i] is the target model's
 * greedy next token after the prefix that ends at node i (slot 0: after the
 * context alone).  Serial greedy decoding emits target[0]; it agrees with
 * the draft exactly when some child of the root carries that token, and so
 * on down the tree ([gist] "Résultats expérimentaux -- Absence de perte";
 * [captcha] "Methodology -- deep read": the longest accepted root-to-leaf
 * path is verified in one forward pass).  Starting from the root, the walk
 * moves to the child of the current node whose token equals the target's
 * token at the current node (children of one node carry distinct tokens;
 * were two equal, the lower slot is taken) and stops at a node with no such
 * child.
 *
 * Outputs: path[0 .. accepted) the accepted slots in order, the rest of
 * path[0 .. n] set to -1; *accepted the number of accepted draft tokens;
 * *bonus the target's token at the last accepted node (the round emits
 * accepted + 1 tokens).  The walk takes at most n steps, so a malformed
 * tree cannot make it loop.
 */
int oracle_accept_greedy(int n, int count, const int32_t *tokens, const int32_t *parents,
                         const int32_t *target, int32_t *path, int32_t *accepted, int32_t *bonus)
{
    if (n < 1 || !tokens || !parents || !target || !path || !accepted || !bonus) return OR_EINVAL;
    if (count < 0) count = 0;
    if (count > n) count = n;
    for (int i = 0; i <= n; ++i) path[i] = -1;
    int u = 0, k = 0;
    while (k < n) {
        int next = -1;
        for (int c = 1; c <= count; ++c) {
            if (parents[c] == u && tokens[c] == target[u]) { next = c; break; }
        }
        if (next < 0) break;
        path[k++] = next;
        u = next;
    }
    *accepted = k;
    *bonus = target[u];
    return OR_OK;
}
