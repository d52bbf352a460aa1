/*
 * oracle_sanitize.c -- runs every entry point of the fp64 CPU oracle on small
 * inputs (every dtype, edge sizes, data errors, broken trees) inside one
 * process built with AddressSanitizer and UndefinedBehaviorSanitizer, so an
 * out-of-bounds access, a leak or undefined arithmetic anywhere in the oracle
 * ends the run with a report.  Test infrastructure: compiled and run by
 * tests/test_sanitize_host.py on the CPU.  The oracle is compiled into this
 * translation unit.
 */
#include "../../oracle/sv_oracle.c"

#include <stdio.h>

static uint64_t g_rng = 0x9E3779B97F4A7C15ull;
static double urand(void)
{
    g_rng ^= g_rng << 13;
    g_rng ^= g_rng >> 7;
    g_rng ^= g_rng << 17;
    return (double)(g_rng >> 11) * (1.0 / 9007199254740992.0);
}

static int g_cases = 0;
#define CHECK(cond)                                                                  \
    do {                                                                             \
        if (!(cond)) {                                                               \
            fprintf(stderr, "check failed at line %d: %s\n", __LINE__, #cond);       \
            exit(2);                                                                 \
        }                                                                            \
    } while (0)

/* rows [n][V] of logits in the given dtype (bf16 as the high half of a float) */
static void* make_rows(int dtype, int64_t n, int V, double scale)
{
    const size_t es = elem_size(dtype);
    void* p = malloc(es * (size_t)(n * V > 0 ? n * V : 1));
    for (int64_t i = 0; i < n * V; ++i) {
        const double z = scale * (2.0 * urand() - 1.0);
        if (dtype == ORC_F64) {
            ((double*)p)[i] = z;
        } else if (dtype == ORC_F32) {
            ((float*)p)[i] = (float)z;
        } else {
            const float f = (float)z;
            uint32_t u;
            memcpy(&u, &f, 4);
            ((uint16_t*)p)[i] = (uint16_t)(u >> 16);
        }
    }
    return p;
}

static void set_logit(void* rows, int dtype, int64_t i, double z)
{
    if (dtype == ORC_F64) {
        ((double*)rows)[i] = z;
    } else if (dtype == ORC_F32) {
        ((float*)rows)[i] = (float)z;
    } else {
        const float f = (float)z;
        uint32_t u;
        memcpy(&u, &f, 4);
        ((uint16_t*)rows)[i] = (uint16_t)(u >> 16);
    }
}

typedef struct {
    int32_t *tokens, *num, *path, *acc, *stop, *kind, *query;
    double *qt, *pt, *ratio, *uacc, *us, *mass, *W, *target, *lo, *hi, *qlo, *qhi, *lq, *lp;
    orc_out o;
} outs;

static void outs_alloc(outs* s, int B, int width, int nslots, int rows, int tree, int V)
{
    memset(s, 0, sizeof(*s));
    s->tokens = calloc((size_t)B * width + 1, 4);
    s->num = calloc((size_t)B + 1, 4);
    s->path = tree ? calloc((size_t)B * width + 1, 4) : NULL;
    s->acc = calloc((size_t)B * nslots + 1, 4);
    s->stop = calloc((size_t)B + 1, 4);
    s->kind = calloc((size_t)B + 1, 4);
    s->query = calloc((size_t)B + 1, 4);
    for (int b = 0; b < B; ++b) s->query[b] = (int32_t)(urand() * V);
    double** d[] = {&s->qt, &s->pt, &s->ratio, &s->uacc};
    for (int i = 0; i < 4; ++i) *d[i] = calloc((size_t)B * nslots + 1, 8);
    double** e[] = {&s->us, &s->mass, &s->W, &s->target, &s->lo, &s->hi, &s->qlo, &s->qhi};
    for (int i = 0; i < 8; ++i) *e[i] = calloc((size_t)B + 1, 8);
    s->lq = calloc((size_t)B * rows + 1, 8);
    s->lp = calloc((size_t)B * rows + 1, 8);
    orc_out o = {s->tokens, s->num, s->path, s->acc, s->qt, s->pt, s->ratio, s->uacc, s->us, s->mass, s->W,
                 s->target, s->lo, s->hi, s->query, s->qlo, s->qhi, s->stop, s->kind, s->lq, s->lp};
    s->o = o;
}

static void outs_free(outs* s)
{
    void* p[] = {s->tokens, s->num, s->path, s->acc, s->stop, s->kind, s->query, s->qt, s->pt, s->ratio,
                 s->uacc, s->us, s->mass, s->W, s->target, s->lo, s->hi, s->qlo, s->qhi, s->lq, s->lp};
    for (size_t i = 0; i < sizeof(p) / sizeof(p[0]); ++i) free(p[i]);
}

static void chain_case(int dtype, int B, int N, int V, double T, int spoil, int with_u)
{
    void* zq = make_rows(dtype, (int64_t)B * (N + 1), V, 4.0);
    void* zp = make_rows(dtype, (int64_t)B * (N > 0 ? N : 1), V, 4.0);
    int32_t* d = malloc(sizeof(int32_t) * (size_t)(B * N + 1));
    for (int i = 0; i < B * N; ++i) d[i] = (int32_t)(urand() * V);
    if (spoil && B > 0) {
        set_logit(zq, dtype, 0, NAN);                                    /* NaN in sequence 0 */
        if (B > 1 && N > 0) d[N] = V + 3;                                 /* token out of range */
        if (B > 2) for (int t = 0; t < V; ++t) set_logit(zq, dtype, (int64_t)2 * (N + 1) * V + t, -INFINITY);
        if (B > 3 && N > 0) set_logit(zp, dtype, (int64_t)3 * N * V + d[3 * N], -INFINITY);
    }
    double* u = NULL;
    if (with_u) {
        u = malloc(sizeof(double) * (size_t)(B * (2 * N + 1) + 1));
        for (int i = 0; i < B * (2 * N + 1); ++i) u[i] = urand();
    }
    outs s;
    outs_alloc(&s, B, N + 1, N > 0 ? N : 1, N + 1, 0, V);
    const int64_t es = 1;
    (void)es;
    int rc = orc_verify_chain(zq, (int64_t)(N + 1) * V, V, zp, (int64_t)(N > 0 ? N : 1) * V, V, dtype, d, B, N, V,
                              7, 3, T, u, 0, B, 2, &s.o);
    CHECK(rc == 0);
    for (int b = 0; b < B; ++b) CHECK(s.num[b] >= -1 && s.num[b] <= N);
    outs_free(&s);
    free(zq);
    free(zp);
    free(d);
    free(u);
    ++g_cases;
}

static void tree_case(int dtype, int B, int Tn, int V, int max_depth, int walk, int shared, int spoil)
{
    const int nn = Tn + 1;
    void* zq = make_rows(dtype, (int64_t)B * nn, V, 3.0);
    void* zp = make_rows(dtype, (int64_t)B * nn, V, 3.0);
    int32_t* tok = malloc(sizeof(int32_t) * (size_t)(B * nn));
    int32_t* par = malloc(sizeof(int32_t) * (size_t)((shared ? 1 : B) * nn));
    for (int i = 0; i < B * nn; ++i) tok[i] = (int32_t)(urand() * V);
    for (int r = 0; r < (shared ? 1 : B); ++r) {
        par[r * nn] = -1;
        for (int n = 1; n < nn; ++n) par[r * nn + n] = (int32_t)(urand() * n);
    }
    if (spoil && nn > 2) {
        par[nn - 1] = nn + 5;           /* parent outside [0, n) */
        if (!shared && B > 1) par[nn + 1] = -3;
        tok[1] = -2;
    }
    const int nu = Tn + max_depth + 1;
    double* u = malloc(sizeof(double) * (size_t)(B * nu + 1));
    for (int i = 0; i < B * nu; ++i) u[i] = urand();
    outs s;
    outs_alloc(&s, B, max_depth + 1, nn, nn, 1, V);
    int rc = orc_verify_tree(zq, (int64_t)nn * V, V, zp, (int64_t)nn * V, V, dtype, tok, par, shared, B, Tn, V,
                             max_depth, walk, 11, 5, 0.8, spoil ? NULL : u, 0, B, 2, &s.o);
    CHECK(rc == 0);
    for (int b = 0; b < B; ++b) CHECK(s.num[b] >= -1 && s.num[b] <= max_depth);
    /* the indices and gather of the walk just taken */
    const int L = nn + max_depth + 4, rb = 16, P = 2;
    int32_t* kvin = malloc(sizeof(int32_t) * (size_t)(B + 1));
    for (int b = 0; b < B; ++b) kvin[b] = (int32_t)(urand() * 4);
    int32_t* src = malloc(sizeof(int32_t) * (size_t)(B * (max_depth + 1) + 1));
    int32_t* kvl = malloc(sizeof(int32_t) * (size_t)(B + 1));
    uint8_t* kv = malloc((size_t)P * B * L * rb + 1);
    for (size_t i = 0; i < (size_t)P * B * L * rb; ++i) kv[i] = (uint8_t)(urand() * 256);
    rc = orc_kv_compact(s.path, s.num, kvin, B, max_depth, src, kvl, kv, (int64_t)L * rb, rb, rb, P,
                        (int64_t)B * L * rb);
    CHECK(rc == 0);
    rc = orc_kv_compact(NULL, s.num, kvin, B, max_depth, src, kvl, NULL, 0, 0, 0, 0, 0);
    CHECK(rc == 0);
    /* the tree's attention mask and positions */
    const int W = (nn + 63) / 64;
    uint64_t* mask = calloc((size_t)B * nn * W + 1, 8);
    int32_t* pos = calloc((size_t)B * nn + 1, 4);
    rc = orc_tree_mask(par, shared, kvin, B, Tn, mask, pos);
    CHECK(rc == 0);
    rc = orc_tree_mask(par, shared, NULL, B, Tn, mask, pos);
    CHECK(rc == 0);
    free(mask);
    free(pos);
    free(kvin);
    free(src);
    free(kvl);
    free(kv);
    outs_free(&s);
    free(zq);
    free(zp);
    free(tok);
    free(par);
    free(u);
    ++g_cases;
}

static void draft_case(int dtype, int B, int R, int V, double T, int spoil)
{
    void* z = make_rows(dtype, (int64_t)B * R, V, 5.0);
    if (spoil && B * R > 0) {
        set_logit(z, dtype, 0, NAN);
        if (B * R > 1) for (int t = 0; t < V; ++t) set_logit(z, dtype, (int64_t)V + t, -INFINITY);
        if (B * R > 2) set_logit(z, dtype, (int64_t)2 * V, INFINITY);
    }
    const size_t n = (size_t)B * R + 1;
    int32_t* tok = malloc(4 * n);
    int32_t* q = malloc(4 * n);
    for (size_t i = 0; i < n; ++i) q[i] = (int32_t)(urand() * V);
    double* f[8];
    for (int i = 0; i < 8; ++i) f[i] = malloc(8 * n);
    int rc = orc_sample_draft(z, (int64_t)R * V, V, dtype, B, R, V, T, 9, 2, 1, NULL, tok, f[0], f[1], f[2], f[3],
                              f[4], f[5], q, f[6], f[7], 2);
    CHECK(rc == 0);
    rc = orc_sample_draft(z, (int64_t)R * V, V, dtype, B, R, V, T, 9, 2, 0, f[1], tok, f[0], NULL, NULL, NULL, NULL,
                          NULL, NULL, NULL, NULL, 1);
    CHECK(rc == 0);
    for (int i = 0; i < 8; ++i) free(f[i]);
    free(tok);
    free(q);
    free(z);
    ++g_cases;
}

static void build_case(int dtype, int B, int V, int depth, int topk, int budget)
{
    const int n_exp = 1 + topk * (depth - 1);
    void* rows = make_rows(dtype, (int64_t)B * n_exp, V, 4.0);
    const int nn = budget + 1;
    int32_t* par = malloc(4 * (size_t)(B * nn));
    int32_t* tok = malloc(4 * (size_t)(B * nn));
    int32_t* dep = malloc(4 * (size_t)(B * nn));
    double* sc = malloc(8 * (size_t)(B * nn));
    int32_t* fr = malloc(4 * (size_t)(B * (depth > 1 ? depth - 1 : 1) * topk));
    int rc = orc_tree_build(rows, (int64_t)n_exp * V, V, dtype, B, V, depth, topk, budget, 1.0, par, tok, dep, sc,
                            fr);
    CHECK(rc == 0);
    for (int i = 0; i < B * nn; ++i) CHECK(par[i] >= -1 && par[i] < nn);
    free(rows);
    free(par);
    free(tok);
    free(dep);
    free(sc);
    free(fr);
    ++g_cases;
}

static void small_fns(void)
{
    const int V = 37;
    for (int dtype = 0; dtype < 3; ++dtype) {
        void* q = make_rows(dtype, 1, V, 3.0);
        void* p = make_rows(dtype, 1, V, 3.0);
        double m, lse;
        CHECK(orc_row_lse(q, dtype, V, 0.7, &m, &lse) == 0);
        double* w = malloc(8 * V);
        CHECK(orc_residual_probs(q, p, dtype, V, 0.7, w) == 0);
        const int t = orc_inverse_cdf(w, V, 0.5);
        CHECK(t >= -1 && t < V);
        (void)orc_accept_prob(q, p, dtype, V, 0.7, 3);
        free(w);
        free(q);
        free(p);
        ++g_cases;
    }
    double w1[1] = {0.0};
    CHECK(orc_inverse_cdf(w1, 1, 0.3) >= -1);
    double ua[6], us[6];
    orc_uniform_grid(1, 2, 2, 3, ua, us);
    uint32_t c[4] = {1, 2, 3, 4}, k[2] = {5, 6}, o[4];
    orc_philox4x32_10(c, k, o);
    ++g_cases;
}

int main(void)
{
#ifdef SANITIZE_SELFTEST
    /* the sanitizer itself: a read one past a heap block must be reported */
    {
        volatile int32_t* probe = malloc(4 * sizeof(int32_t));
        probe[0] = 1;
        printf("%d\n", (int)probe[4]);
        free((void*)probe);
    }
#endif
    const int dts[3] = {ORC_F32, ORC_BF16, ORC_F64};
    for (int i = 0; i < 3; ++i) {
        const int dt = dts[i];
        chain_case(dt, 4, 3, 50, 1.0, 0, 0);
        chain_case(dt, 5, 2, 41, 0.6, 1, 1);
        chain_case(dt, 3, 0, 17, 1.3, 0, 0);   /* no drafts: bonus only */
        chain_case(dt, 2, 64, 9, 1.0, 0, 0);   /* the longest chain */
        chain_case(dt, 2, 1, 1, 2.0, 0, 1);    /* V = 1 */
        chain_case(dt, 0, 3, 8, 1.0, 0, 0);    /* empty batch */
        tree_case(dt, 3, 9, 33, 4, 0, 1, 0);
        tree_case(dt, 3, 9, 33, 4, 1, 0, 0);
        tree_case(dt, 2, 7, 21, 3, 0, 0, 1);   /* broken parents, bad token */
        tree_case(dt, 2, 0, 12, 0, 0, 1, 0);   /* root only */
        tree_case(dt, 1, 70, 15, 70, 1, 1, 0); /* two mask words */
        draft_case(dt, 3, 4, 29, 0.9, 0);
        draft_case(dt, 2, 3, 19, 1.1, 1);
        draft_case(dt, 1, 1, 1, 1.0, 0);
        build_case(dt, 2, 40, 3, 4, 10);
        build_case(dt, 1, 16, 1, 16, 16);
    }
    small_fns();
    /* arguments the oracle refuses */
    outs s;
    outs_alloc(&s, 1, 2, 1, 2, 0, 4);
    CHECK(orc_verify_chain(NULL, 0, 0, NULL, 0, 0, 0, NULL, 1, 1, 0, 0, 0, 1.0, NULL, 0, 1, 1, &s.o) == 1);
    CHECK(orc_verify_chain(NULL, 0, 0, NULL, 0, 0, 0, NULL, 1, 1, 4, 0, 0, 0.0, NULL, 0, 1, 1, &s.o) == 1);
    outs_free(&s);
    CHECK(orc_tree_build(NULL, 0, 0, 0, 1, 10, 2, 11, 5, 1.0, NULL, NULL, NULL, NULL, NULL) == 1);
    CHECK(orc_tree_build(NULL, 0, 0, 0, 1, 10, 2, 2, 99, 1.0, NULL, NULL, NULL, NULL, NULL) == 1);
    CHECK(orc_tree_mask(NULL, 1, NULL, -1, 3, NULL, NULL) == 1);
    CHECK(orc_kv_compact(NULL, NULL, NULL, -1, 2, NULL, NULL, NULL, 0, 0, 0, 0, 0) == 1);
    printf("oracle sanitize: %d cases clean\n", g_cases);
    return 0;
}
