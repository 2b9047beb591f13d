/*
 * oracle_sanitize_check.c -- runs every entry point of the CPU oracle
 * (oracle/dtree_oracle.c) on small inputs, valid and invalid, so that a build
 * with AddressSanitizer and UndefinedBehaviorSanitizer can report any
 * out-of-bounds access, leak or undefined operation in it.
 *
 * Test infrastructure: built and run by tests/test_sanitizers.py.  Inputs come
 * from a 64-bit linear congruential generator (no method arithmetic here);
 * the checks are on return codes and on structural properties only -- the
 * oracle's values are pinned elsewhere.  Exit status 0 = every check passed.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

int oracle_topm_row(const void *row, int dtype, int V, int M, int32_t *idx, double *val);
int oracle_tail_lse(const void *row, int dtype, int V, int M, double T, const int32_t *idx, double *out);
int oracle_gru(const void *xmat, int64_t xrow, int dtype, const double *h, const void *W_ih, const void *W_hh,
               const void *b_ih, const void *b_hh, int E, int H, double *h_out);
int oracle_dist(const int32_t *idx, const double *val, int M, const void *C, int dtype, int H, const double *h,
                double T, double tail, int32_t *tok_sorted, double *lp_sorted);
int oracle_build_request(int V, int L, int E, int H, int M, int n, double T, int dtype, double eps,
                         const void *base, const void *emb, const void *W_ih, const void *W_hh,
                         const void *b_ih, const void *b_hh, const void *C, const float *h0, int32_t *tokens,
                         int32_t *parents, int32_t *depths, double *scores, uint8_t *mask, int32_t *count,
                         uint32_t *flags, double *min_gap, int32_t *topm_idx, double *topm_val, int full_vocab,
                         double *tail_out, int32_t *first_flag);
int oracle_score_paths(int V, int L, int E, int H, int M, double T, int dtype, const void *base, const void *emb,
                       const void *W_ih, const void *W_hh, const void *b_ih, const void *b_hh, const void *C,
                       const float *h0, int npaths, const int32_t *paths, const int32_t *len, double *out,
                       int full_vocab);
int oracle_accept_greedy(int n, int count, const int32_t *tokens, const int32_t *parents, const int32_t *target,
                         int32_t *path, int32_t *accepted, int32_t *bonus);

static int failures = 0;
#define CHECK(cond)                                                          \
    do {                                                                     \
        if (!(cond)) {                                                       \
            fprintf(stderr, "check failed at line %d: %s\n", __LINE__, #cond); \
            ++failures;                                                      \
        }                                                                    \
    } while (0)

static uint64_t rng_state = 0x9E3779B97F4A7C15ull;
static double uniform(void) /* [-1, 1) */
{
    rng_state = rng_state * 6364136223846793005ull + 1442695040888963407ull;
    return (double)(rng_state >> 11) * (2.0 / 9007199254740992.0) - 1.0;
}

/* an array of n inputs in the requested storage type (0: binary32, 1: bf16 bits) */
static void *make(int dtype, size_t n, double scale)
{
    if (dtype == 0) {
        float *p = (float *)malloc(n * sizeof *p);
        for (size_t i = 0; i < n; ++i) p[i] = (float)(scale * uniform());
        return p;
    }
    uint16_t *p = (uint16_t *)malloc(n * sizeof *p);
    for (size_t i = 0; i < n; ++i) {
        float f = (float)(scale * uniform());
        uint32_t u;
        memcpy(&u, &f, sizeof u);
        p[i] = (uint16_t)(u >> 16);
    }
    return p;
}

/* one whole build, its structure checked */
static void build_case(int V, int L, int E, int H, int M, int n, double T, int dtype, int full_vocab, int biases,
                       int with_h0)
{
    void *base = make(dtype, (size_t)L * V, 4.0), *emb = make(dtype, (size_t)V * E, 0.2);
    void *wih = make(dtype, (size_t)3 * H * E, 0.2), *whh = make(dtype, (size_t)3 * H * H, 0.2);
    void *bih = biases ? make(dtype, (size_t)3 * H, 0.1) : NULL, *bhh = biases ? make(dtype, (size_t)3 * H, 0.1) : NULL;
    void *C = make(dtype, (size_t)V * H, 0.5);
    float *h0 = with_h0 ? (float *)make(0, (size_t)H, 1.0) : NULL;
    const int S = n + 1;
    int32_t *tok = malloc(S * sizeof *tok), *par = malloc(S * sizeof *par), *dep = malloc(S * sizeof *dep);
    double *sc = malloc(S * sizeof *sc), gap = 0.0;
    uint8_t *mask = malloc((size_t)S * S);
    int32_t cnt = -1, first = -1;
    uint32_t flags = 0;
    int32_t *tidx = malloc((size_t)L * M * sizeof *tidx);
    double *tval = malloc((size_t)L * M * sizeof *tval), *tail = malloc((size_t)L * sizeof *tail);
    int rc = oracle_build_request(V, L, E, H, M, n, T, dtype, 1e-5, base, emb, wih, whh, bih, bhh, C, h0, tok, par,
                                  dep, sc, mask, &cnt, &flags, &gap, tidx, tval, full_vocab, tail, &first);
    CHECK(rc == 0);
    CHECK(cnt >= 1 && cnt <= n);
    CHECK(first >= 0 && first <= cnt);
    for (int v = 1; v <= cnt; ++v) {
        CHECK(par[v] >= 0 && par[v] < v);
        CHECK(dep[v] == dep[par[v]] + 1 && dep[v] <= L);
        CHECK(sc[v] <= sc[par[v]]);
    }
    /* every node path rescored on its own */
    int32_t *paths = calloc((size_t)(cnt > 0 ? cnt : 1) * L, sizeof *paths);
    int32_t *len = calloc((size_t)(cnt > 0 ? cnt : 1), sizeof *len);
    double *out = calloc((size_t)(cnt > 0 ? cnt : 1), sizeof *out);
    for (int v = 1; v <= cnt; ++v) {
        len[v - 1] = dep[v];
        for (int j = v; j > 0; j = par[j]) paths[(size_t)(v - 1) * L + dep[j] - 1] = tok[j];
    }
    rc = oracle_score_paths(V, L, E, H, M, T, dtype, base, emb, wih, whh, bih, bhh, C, h0, cnt, paths, len, out,
                            full_vocab);
    CHECK(rc == 0);
    for (int v = 1; v <= cnt; ++v) CHECK(out[v - 1] == sc[v]);
    /* the acceptance walk over the built tree, every slot's target its first child's token */
    int32_t *target = malloc(S * sizeof *target), *path = malloc(S * sizeof *path), acc = -1, bonus = -1;
    for (int i = 0; i < S; ++i) target[i] = (int32_t)(i * 7 % V);
    for (int v = cnt; v >= 1; --v) target[par[v]] = tok[v];
    rc = oracle_accept_greedy(n, cnt, tok, par, target, path, &acc, &bonus);
    CHECK(rc == 0 && acc >= 1 && acc <= cnt);
    free(base); free(emb); free(wih); free(whh); free(bih); free(bhh); free(C); free(h0);
    free(tok); free(par); free(dep); free(sc); free(mask); free(tidx); free(tval); free(tail);
    free(paths); free(len); free(out); free(target); free(path);
}

int main(void)
{
    /* top-M of rows with exact ties, M = V and V = 1 */
    for (int dtype = 0; dtype < 2; ++dtype) {
        const int V = 37;
        void *row = make(dtype, V, 2.0);
        int32_t idx[37];
        double val[37], tail = 0.0;
        CHECK(oracle_topm_row(row, dtype, V, 5, idx, val) == 0);
        CHECK(oracle_topm_row(row, dtype, V, V, idx, val) == 0);
        CHECK(oracle_tail_lse(row, dtype, V, V, 0.0, idx, &tail) == 0 && isinf(tail) && tail < 0);
        CHECK(oracle_topm_row(row, dtype, V, 8, idx, val) == 0);
        CHECK(oracle_tail_lse(row, dtype, V, 8, 0.5, idx, &tail) == 0 && isfinite(tail));
        CHECK(oracle_topm_row(row, dtype, 1, 1, idx, val) == 0 && idx[0] == 0);
        CHECK(oracle_topm_row(row, dtype, V, V + 1, idx, val) != 0); /* M > V */
        CHECK(oracle_topm_row(NULL, dtype, V, 4, idx, val) != 0);
        int32_t bad[8] = {0, 1, 2, 3, 4, 5, 6, 99};
        CHECK(oracle_tail_lse(row, dtype, V, 8, 0.0, bad, &tail) != 0); /* id outside the row */
        free(row);
    }
    /* one GRU step and one children distribution, with and without biases */
    {
        const int E = 12, H = 8, V = 20, M = 6;
        void *x = make(1, (size_t)V * E, 0.5), *wih = make(1, (size_t)3 * H * E, 0.3), *whh = make(1, (size_t)3 * H * H, 0.3);
        void *b = make(1, (size_t)3 * H, 0.1), *C = make(1, (size_t)V * H, 0.5);
        double h[8], ho[8], val[6], lp[6];
        int32_t idx[6] = {3, 1, 4, 15, 9, 2}, tok[6];
        for (int k = 0; k < H; ++k) h[k] = uniform();
        for (int j = 0; j < M; ++j) val[j] = uniform();
        CHECK(oracle_gru(x, V - 1, 1, h, wih, whh, b, b, E, H, ho) == 0);
        CHECK(oracle_gru(x, 0, 1, h, wih, whh, NULL, NULL, E, H, ho) == 0);
        CHECK(oracle_gru(x, -1, 1, h, wih, whh, NULL, NULL, E, H, ho) != 0);
        for (int k = 0; k < H; ++k) CHECK(fabs(ho[k]) < 1.0 + fabs(h[k]));
        CHECK(oracle_dist(idx, val, M, C, 1, H, h, 0.0, -INFINITY, tok, lp) == 0);
        for (int j = 1; j < M; ++j) CHECK(lp[j] <= lp[j - 1]);
        CHECK(oracle_dist(idx, val, M, C, 1, H, h, 0.7, 1.5, tok, lp) == 0);
        CHECK(oracle_dist(idx, val, M, C, 1, H, h, -1.0, -INFINITY, tok, lp) != 0);
        free(x); free(wih); free(whh); free(b); free(C);
    }
    /* whole builds: both dtypes, full-vocabulary mode, temperature, the
     * budget and depth limits, biases and h0 present or not */
    build_case(50, 6, 8, 8, 5, 16, 0.0, 0, 0, 1, 0);
    build_case(50, 6, 8, 8, 5, 16, 0.5, 1, 1, 0, 1);
    build_case(64, 8, 16, 8, 8, 64, 0.0, 1, 0, 1, 1);
    build_case(30, 1, 4, 4, 7, 5, 0.0, 0, 0, 0, 0);   /* L = 1 */
    build_case(30, 4, 4, 4, 1, 9, 0.0, 0, 1, 1, 0);   /* M = 1: a chain */
    build_case(30, 4, 4, 4, 30, 1, 1.0, 1, 0, 1, 1);  /* n = 1, M = V */
    /* invalid builds return an error */
    {
        int32_t tok[3], par[3], dep[3], cnt, first;
        double sc[3], gap;
        uint8_t mask[9];
        uint32_t flags;
        float dummy[64] = {0};
        CHECK(oracle_build_request(10, 2, 2, 2, 11, 2, 0.0, 0, 1e-5, dummy, dummy, dummy, dummy, NULL, NULL, dummy,
                                   NULL, tok, par, dep, sc, mask, &cnt, &flags, &gap, NULL, NULL, 0, NULL,
                                   &first) != 0); /* M > V */
        CHECK(oracle_build_request(10, 2, 2, 2, 3, 2, 0.0, 5, 1e-5, dummy, dummy, dummy, dummy, NULL, NULL, dummy,
                                   NULL, tok, par, dep, sc, mask, &cnt, &flags, &gap, NULL, NULL, 0, NULL,
                                   NULL) != 0); /* unknown dtype */
        int32_t target[3] = {0, 0, 0}, path[3], acc, bonus;
        CHECK(oracle_accept_greedy(0, 0, tok, par, target, path, &acc, &bonus) != 0);
    }
    if (failures) {
        fprintf(stderr, "%d checks failed\n", failures);
        return 1;
    }
    printf("oracle sanitizer check: all entry points ran clean\n");
    return 0;
}
