/*
 * sv_oracle.c -- plain, slow, obviously-correct fp64 CPU oracle of the
 * speculative-decoding verify-and-accept step (Leviathan rejection sampling,
 * chain and EAGLE-style draft tree) plus the KV-compaction indices/gather.
 *
 * TEST INFRASTRUCTURE ONLY.  The test-suite, the smoke check and the CPU
 * baseline leg of the benchmark are the only code that may load this
 * library.  It shares no source, header, table or helper with the HIP
 * library, and the HIP library never falls back to it.
 *
 * Pages followed (cited by title and section):
 *   [PT] "Decodificacao Especulativa e EAGLE-3", ai-engineering.academy,
 *        Fase 10 - Licao 15.
 *   [FA] the same lesson in Persian, nextadmin.net, "Speculative decoding and
 *        EAGLE-3: optimising LLM inference speed".
 *   [ZH] "投机解码与 EAGLE：步骤、发展历史与三代差异", caijizhuo.github.io.
 *
 * Notation: q = verifier (target) distribution, p = draft distribution, as in
 * [PT] "O Conceito / O invariante" ([ZH] swaps the two letters).
 *
 * Precision: every quantity is an IEEE double; bf16 and fp32 inputs widen to
 * double exactly; exp/log are the host libm's.  Loops are sequential; the
 * only parallelism is OpenMP across independent sequences.
 *
 * Readings taken where the pages are silent (each is also listed in the
 * design notes of the repository):
 *   R1  temperature T > 0 divides both q- and p-logits before the softmax.
 *   R2  the accept ratio q(d)/p(d) is formed in the log domain, so the
 *       "draft probability <= 0 -> accept" branch fires only for a draft
 *       logit of -inf.
 *   R3  sample() is an inverse CDF in token-id order over unnormalised
 *       weights: the first token whose running sum exceeds u*W; if rounding
 *       leaves none, the last token of positive weight.
 *   R4  uniforms: Philox4x32-10, key = seed, counter = (position, sequence,
 *       round low word, (round high word << 4) | stream); the accept uniform
 *       of position/node n is the 53-bit double made from output words 0,1 of
 *       the block at position n, the sampling uniform of slot s is the one
 *       made from words 2,3 of the block at position s.
 *   R5  tree: node n >= 1 is tested with q/p at parent(n); the walk descends
 *       into the lowest-index accepted child, stops at a leaf (bonus from the
 *       leaf's q) or at a node with no accepted child (residual of that
 *       node's q and p), and never appends a bonus after a rejection.
 *   R5b the pages' literal walk ([ZH] section 4, "eagle_round" step 4: take
 *       the node's best child, accept and descend, or reject, resample and
 *       end): the best child is the lowest-index child (siblings come in
 *       descending draft probability); the walk stops with the residual of
 *       the node's q and p as soon as that child is rejected, whatever its
 *       siblings' decisions.  Selected by walk = 1.
 *   R6  data errors (NaN or +inf in a row the outcome reads, a row that is
 *       all -inf, a token outside [0,V), a parent not in [0,n), a walk longer
 *       than max_depth) mark the sequence with num_accepted = -1.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

enum { ORC_F32 = 0, ORC_BF16 = 1, ORC_F64 = 2 };
enum { KIND_RESIDUAL = 0, KIND_BONUS = 1, KIND_RESIDUAL_WAS_ZERO = 2, KIND_ERROR = -1 };

/* ------------------------------------------------------------------------- */
/* Philox4x32-10: Salmon, Moraes, Dror, Shaw, "Parallel random numbers: as    */
/* easy as 1, 2, 3", SC'11.  Ten rounds of the 4x32 S-box; the key is bumped  */
/* by the Weyl constants before every round but the first.                   */
/* ------------------------------------------------------------------------- */
void orc_philox4x32_10(const uint32_t ctr_in[4], const uint32_t key_in[2], uint32_t out[4])
{
    uint32_t c0 = ctr_in[0], c1 = ctr_in[1], c2 = ctr_in[2], c3 = ctr_in[3];
    uint32_t k0 = key_in[0], k1 = key_in[1];
    for (int r = 0; r < 10; ++r) {
        if (r > 0) {
            k0 += 0x9E3779B9u; /* golden ratio */
            k1 += 0xBB67AE85u; /* sqrt(3) - 1 */
        }
        uint64_t prod_a = (uint64_t)0xD2511F53u * (uint64_t)c0;
        uint64_t prod_b = (uint64_t)0xCD9E8D57u * (uint64_t)c2;
        uint32_t a_hi = (uint32_t)(prod_a >> 32), a_lo = (uint32_t)prod_a;
        uint32_t b_hi = (uint32_t)(prod_b >> 32), b_lo = (uint32_t)prod_b;
        uint32_t n0 = b_hi ^ c1 ^ k0;
        uint32_t n1 = b_lo;
        uint32_t n2 = a_hi ^ c3 ^ k1;
        uint32_t n3 = a_lo;
        c0 = n0; c1 = n1; c2 = n2; c3 = n3;
    }
    out[0] = c0; out[1] = c1; out[2] = c2; out[3] = c3;
}

/* 53-bit uniform in [0,1) from two 32-bit words: the top 27 bits of a and the
 * top 26 bits of b (the construction of Matsumoto and Nishimura's
 * genrand_res53).  Every value is an exact dyadic double. */
double orc_u53(uint32_t a, uint32_t b)
{
    double hi = (double)(a >> 5);
    double lo = (double)(b >> 6);
    return (hi * 67108864.0 + lo) * (1.0 / 9007199254740992.0);
}

/* Block of the verify stream (R4). */
void orc_philox_block(uint64_t seed, uint64_t round, uint32_t seq, uint32_t pos, uint32_t stream,
                      uint32_t out[4])
{
    uint32_t ctr[4], key[2];
    ctr[0] = pos;
    ctr[1] = seq;
    ctr[2] = (uint32_t)round;
    ctr[3] = ((uint32_t)(round >> 32) << 4) | (stream & 15u);
    key[0] = (uint32_t)seed;
    key[1] = (uint32_t)(seed >> 32);
    orc_philox4x32_10(ctr, key, out);
}

/* Accept uniform of position/node `pos` and sampling uniform of slot `pos`. */
void orc_uniforms(uint64_t seed, uint64_t round, uint32_t seq, uint32_t pos, double* u_acc, double* u_samp)
{
    uint32_t w[4];
    orc_philox_block(seed, round, seq, pos, 0u, w);
    if (u_acc) *u_acc = orc_u53(w[0], w[1]);
    if (u_samp) *u_samp = orc_u53(w[2], w[3]);
}

/* Both uniforms of positions 1..npos of sequences 0..nseq-1, row-major
 * [nseq, npos]; either output may be NULL. */
void orc_uniform_grid(uint64_t seed, uint64_t round, int nseq, int npos, double* u_acc, double* u_samp)
{
    for (int s = 0; s < nseq; ++s)
        for (int p = 0; p < npos; ++p) {
            int64_t at = (int64_t)s * npos + p;
            orc_uniforms(seed, round, (uint32_t)s, (uint32_t)(p + 1), u_acc ? &u_acc[at] : NULL,
                         u_samp ? &u_samp[at] : NULL);
        }
}

/* ------------------------------------------------------------------------- */
/* Logit access                                                               */
/* ------------------------------------------------------------------------- */
static double logit_at(const void* row, int dtype, int64_t t)
{
    if (dtype == ORC_F32) return (double)((const float*)row)[t];
    if (dtype == ORC_BF16) {
        uint32_t bits = (uint32_t)((const uint16_t*)row)[t] << 16;
        float f;
        memcpy(&f, &bits, sizeof f);
        return (double)f;
    }
    return ((const double*)row)[t];
}

static size_t elem_size(int dtype) { return dtype == ORC_F32 ? 4 : dtype == ORC_BF16 ? 2 : 8; }

static const void* row_ptr(const void* base, int dtype, int64_t seq_stride, int64_t row_stride, int64_t b,
                           int64_t r)
{
    return (const char*)base + (size_t)(b * seq_stride + r * row_stride) * elem_size(dtype);
}

/* Log-softmax normaliser of one row at temperature T ([PT] "O Conceito": the
 * verifier returns a distribution q at every position; R1).  x_t = z_t / T,
 * m = max x, lse = m + log(sum exp(x_t - m)).  Returns nonzero for a data
 * error (R6). */
int orc_row_lse(const void* row, int dtype, int V, double T, double* m_out, double* lse_out)
{
    double m = -INFINITY;
    for (int t = 0; t < V; ++t) {
        double x = logit_at(row, dtype, t) / T;
        if (isnan(x) || x == INFINITY) return 1;
        if (x > m) m = x;
    }
    if (m == -INFINITY) return 1;
    double s = 0.0;
    for (int t = 0; t < V; ++t) s += exp(logit_at(row, dtype, t) / T - m);
    if (m_out) *m_out = m;
    if (lse_out) *lse_out = m + log(s);
    return 0;
}

/* Probability of every token of a row: q_t = exp(x_t - lse). */
static void row_probs(const void* row, int dtype, int V, double T, double lse, double* out)
{
    for (int t = 0; t < V; ++t) out[t] = exp(logit_at(row, dtype, t) / T - lse);
}

/* ------------------------------------------------------------------------- */
/* The accept rule ([PT] Implementando, Passo 1; [PT] O Conceito): accept the */
/* draft token d when u < min(1, q(d)/p(d)); a draft token of zero draft      */
/* probability is accepted.  Ratio formed in the log domain (R2).             */
/* ------------------------------------------------------------------------- */
static int accept_token(double xq_d, double lse_q, double xp_d, double lse_p, double u, double* q_tok,
                        double* p_tok, double* ratio)
{
    double lq = xq_d - lse_q;
    double lp = xp_d - lse_p;
    *q_tok = exp(lq);
    *p_tok = exp(lp);
    if (xp_d == -INFINITY) {
        *ratio = INFINITY;
        return 1;
    }
    double r = exp(lq - lp);
    *ratio = r;
    double threshold = r < 1.0 ? r : 1.0;
    return u < threshold;
}

/* ------------------------------------------------------------------------- */
/* Residual distribution ([PT] Implementando, Passo 2): w_t = max(0, q_t-p_t);*/
/* if every w_t is zero the distribution falls back to q.  Returns the kind.  */
/* ------------------------------------------------------------------------- */
static int residual_weights(const void* qrow, double lse_q, const void* prow, double lse_p, int dtype, int V,
                            double T, double* w, double* resid_mass)
{
    double s = 0.0;
    for (int t = 0; t < V; ++t) {
        double qt = exp(logit_at(qrow, dtype, t) / T - lse_q);
        double pt = exp(logit_at(prow, dtype, t) / T - lse_p);
        double d = qt - pt;
        w[t] = d > 0.0 ? d : 0.0;
        s += w[t];
    }
    *resid_mass = s;
    if (s == 0.0) {
        row_probs(qrow, dtype, V, T, lse_q, w);
        return KIND_RESIDUAL_WAS_ZERO;
    }
    return KIND_RESIDUAL;
}

/* Inverse CDF in token order (R3).  Writes the total W, the threshold u*W and
 * the running sums just before and just after the chosen token. */
static int inverse_cdf(const double* w, int V, double u, double* W_out, double* target_out, double* lo,
                       double* hi)
{
    double W = 0.0;
    for (int t = 0; t < V; ++t) W += w[t];
    double target = u * W;
    double cum = 0.0;
    int chosen = -1, last_pos = -1;
    double last_lo = 0.0, last_hi = 0.0;
    for (int t = 0; t < V; ++t) {
        double before = cum;
        cum += w[t];
        if (w[t] > 0.0) {
            last_pos = t;
            last_lo = before;
            last_hi = cum;
        }
        if (cum > target) {
            chosen = t;
            *lo = before;
            *hi = cum;
            break;
        }
    }
    if (chosen < 0) {
        chosen = last_pos;
        *lo = last_lo;
        *hi = last_hi;
    }
    *W_out = W;
    *target_out = target;
    return chosen;
}

/* Running sums just before and just after token g (for classifying a token
 * that differs from the oracle's). */
static void cdf_edges(const double* w, int V, int g, double* lo, double* hi)
{
    double cum = 0.0;
    for (int t = 0; t < V && t < g; ++t) cum += w[t];
    *lo = cum;
    *hi = (g >= 0 && g < V) ? cum + w[g] : cum;
}

/* ------------------------------------------------------------------------- */
/* Output block shared by the chain and tree entry points.  Every pointer is */
/* optional except tokens and num_accepted.                                   */
/* ------------------------------------------------------------------------- */
typedef struct {
    void* tokens;       /* int32 [B, N+1] chain / [B, max_depth+1] tree */
    void* num_accepted; /* int32 [B] */
    void* path_nodes;   /* int32 [B, max_depth+1] tree only */
    void* accept;       /* int32 [B, N] chain / [B, T+1] tree (node 0 reads 1) */
    void* q_tok;        /* double, same shape as accept */
    void* p_tok;        /* double */
    void* ratio;        /* double */
    void* u_acc;        /* double */
    void* u_samp;       /* double [B] */
    void* resid_mass;   /* double [B]: sum (q-p)_+ on a rejection, else 0 */
    void* weight_total; /* double [B]: W of the distribution sampled from */
    void* target;       /* double [B]: u_samp * W */
    void* edge_lo;      /* double [B] */
    void* edge_hi;      /* double [B] */
    void* query;        /* const int32 [B]: another token to give edges for */
    void* qedge_lo;     /* double [B] */
    void* qedge_hi;     /* double [B] */
    void* stop_node;    /* int32 [B]: chain k, tree node where the walk stopped */
    void* sample_kind;  /* int32 [B] */
    void* lse_q;        /* double [B, rows]: lse of each q row computed (NaN if not computed) */
    void* lse_p;        /* double [B, rows] */
} orc_out;

#define OUT_I32(o, f, i, v) do { if ((o)->f) ((int32_t*)(o)->f)[i] = (v); } while (0)
#define OUT_F64(o, f, i, v) do { if ((o)->f) ((double*)(o)->f)[i] = (v); } while (0)

static void mark_error(const orc_out* o, int64_t b, int width)
{
    OUT_I32(o, num_accepted, b, -1);
    for (int i = 0; i < width; ++i) OUT_I32(o, tokens, b * width + i, -1);
    if (o->path_nodes)
        for (int i = 0; i < width; ++i) OUT_I32(o, path_nodes, b * width + i, -1);
    OUT_I32(o, sample_kind, b, KIND_ERROR);
    OUT_I32(o, stop_node, b, -1);
}

/* Sample from the residual of (q_row, p_row) or, when p_row is NULL, from
 * q_row itself (the bonus), and fill the sampling outputs.  Returns the
 * token, or -1 on a data error in a row read only here. */
static int sample_at(const orc_out* o, int64_t b, const void* qrow, double lse_q, int q_ok, const void* prow,
                     double lse_p, int dtype, int V, double T, double u)
{
    double* w = (double*)malloc(sizeof(double) * (size_t)(V > 0 ? V : 1));
    int kind;
    double resid = 0.0;
    if (!q_ok) {
        if (orc_row_lse(qrow, dtype, V, T, NULL, &lse_q) != 0) {
            free(w);
            return -1;
        }
    }
    if (prow) {
        kind = residual_weights(qrow, lse_q, prow, lse_p, dtype, V, T, w, &resid);
    } else {
        row_probs(qrow, dtype, V, T, lse_q, w);
        kind = KIND_BONUS;
    }
    double W, target, lo, hi;
    int tok = inverse_cdf(w, V, u, &W, &target, &lo, &hi);
    OUT_F64(o, u_samp, b, u);
    OUT_F64(o, resid_mass, b, prow ? resid : 0.0);
    OUT_F64(o, weight_total, b, W);
    OUT_F64(o, target, b, target);
    OUT_F64(o, edge_lo, b, lo);
    OUT_F64(o, edge_hi, b, hi);
    OUT_I32(o, sample_kind, b, kind);
    if (o->query) {
        int g = ((const int32_t*)o->query)[b];
        double qlo, qhi;
        cdf_edges(w, V, g, &qlo, &qhi);
        OUT_F64(o, qedge_lo, b, qlo);
        OUT_F64(o, qedge_hi, b, qhi);
    }
    free(w);
    return tok;
}

/* ------------------------------------------------------------------------- */
/* Draft-token sampling ([PT] O Conceito and Implementando, Passo 1: the     */
/* draft proposes d ~ p, the draft's distribution; [ZH] section 2 draws each */
/* draft token from the draft model's softmax in turn).  Row r of sequence b */
/* (at zp + (b*seq_stride + r*row_stride) elements) gives one token drawn   */
/* from softmax(z / T) by the inverse CDF of R3 with the uniform of R4's     */
/* block (seed, round, sequence b, position pos0 + r, stream 1), words 0 and */
/* 1.  u_in [B, R] (optional) replaces the uniforms.  Outputs [B, R]: token  */
/* (-1 on a bad row, R6), ln p(token) (NaN on a bad row), the uniform, the   */
/* target u*W, W, the CDF edges of the token drawn, and (with query) of the  */
/* query token.                                                             */
/* ------------------------------------------------------------------------- */
int orc_sample_draft(const void* zp, int64_t seq_stride, int64_t row_stride, int dtype, int B, int R, int V,
                     double T, uint64_t seed, uint64_t round, int pos0, const double* u_in, int32_t* tokens,
                     double* logprob, double* u_out, double* target_out, double* W_out, double* lo_out,
                     double* hi_out, const int32_t* query, double* qlo_out, double* qhi_out, int nthreads)
{
    if (B < 0 || R < 0 || V <= 0 || !(T > 0.0) || pos0 < 0 || !tokens) return 1;
#ifdef _OPENMP
    if (nthreads < 1) nthreads = 1;
#pragma omp parallel for schedule(dynamic, 1) num_threads(nthreads)
#endif
    for (int64_t i = 0; i < (int64_t)B * R; ++i) {
        const int b = (int)(i / R), r = (int)(i % R);
        const void* row = row_ptr(zp, dtype, seq_stride, row_stride, b, r);
        double u;
        if (u_in) {
            u = u_in[i];
        } else {
            uint32_t w4[4];
            orc_philox_block(seed, round, (uint32_t)b, (uint32_t)(pos0 + r), 1u, w4);
            u = orc_u53(w4[0], w4[1]);
        }
        if (u_out) u_out[i] = u;
        double lse;
        if (orc_row_lse(row, dtype, V, T, NULL, &lse) != 0) {
            tokens[i] = -1;
            if (logprob) logprob[i] = NAN;
            continue;
        }
        double* w = (double*)malloc(sizeof(double) * (size_t)V);
        row_probs(row, dtype, V, T, lse, w);
        double W, target, lo, hi;
        const int tok = inverse_cdf(w, V, u, &W, &target, &lo, &hi);
        tokens[i] = tok;
        if (logprob) logprob[i] = tok >= 0 ? logit_at(row, dtype, tok) / T - lse : NAN;
        if (target_out) target_out[i] = target;
        if (W_out) W_out[i] = W;
        if (lo_out) lo_out[i] = lo;
        if (hi_out) hi_out[i] = hi;
        if (query && qlo_out && qhi_out) {
            double qlo = NAN, qhi = NAN;
            if (query[i] >= 0 && query[i] < V) cdf_edges(w, V, query[i], &qlo, &qhi);
            qlo_out[i] = qlo;
            qhi_out[i] = qhi;
        }
        free(w);
    }
    return 0;
}

/* ------------------------------------------------------------------------- */
/* Chain verify ([PT] O Conceito: N stacked accept calls, left to right; at */
/* the first rejection at position j sample residual(q_j, p_j) and stop; if  */
/* everything is accepted, a bonus token from q_{N+1}.  [ZH] section 2 and   */
/* section 4 "spec_decode" describe the same loop).                          */
/*                                                                           */
/* zq: [B, N+1, V] rows of q (row i is the distribution that tests d_{i+1}),  */
/* zp: [B, N, V] rows of p, d: [B, N] draft tokens.  u_in (optional) gives    */
/* per sequence 2N+1 uniforms: the accept uniforms of positions 1..N, then   */
/* the sampling uniforms of slots 1..N+1; NULL draws them from Philox (R4).  */
/* ------------------------------------------------------------------------- */
int orc_verify_chain(const void* zq, int64_t q_seq_stride, int64_t q_row_stride, const void* zp,
                     int64_t p_seq_stride, int64_t p_row_stride, int dtype, const int32_t* d, int B, int N, int V,
                     uint64_t seed, uint64_t round, double T, const double* u_in, int b_begin, int b_end,
                     int nthreads, orc_out* o)
{
    if (B < 0 || N < 0 || V <= 0 || !(T > 0.0) || b_begin < 0 || b_end > B || !o || !o->tokens ||
        !o->num_accepted)
        return 1;
#ifdef _OPENMP
    if (nthreads < 1) nthreads = 1;
#pragma omp parallel for schedule(dynamic, 1) num_threads(nthreads)
#endif
    for (int b = b_begin; b < b_end; ++b) {
        const int width = N + 1;
        int err = 0;
        double* lse_q = (double*)malloc(sizeof(double) * (size_t)(N + 1));
        double* lse_p = (double*)malloc(sizeof(double) * (size_t)(N > 0 ? N : 1));
        for (int i = 0; i <= N; ++i) {
            OUT_F64(o, lse_q, (int64_t)b * (N + 1) + i, NAN);
            if (i < N) OUT_F64(o, lse_p, (int64_t)b * (N + 1) + i, NAN);
        }
        /* statistics of the 2N rows the accept tests read */
        for (int i = 0; i < N && !err; ++i) {
            const void* qr = row_ptr(zq, dtype, q_seq_stride, q_row_stride, b, i);
            const void* pr = row_ptr(zp, dtype, p_seq_stride, p_row_stride, b, i);
            if (orc_row_lse(qr, dtype, V, T, NULL, &lse_q[i]) != 0) err = 1;
            if (!err && orc_row_lse(pr, dtype, V, T, NULL, &lse_p[i]) != 0) err = 1;
            if (!err) {
                OUT_F64(o, lse_q, (int64_t)b * (N + 1) + i, lse_q[i]);
                OUT_F64(o, lse_p, (int64_t)b * (N + 1) + i, lse_p[i]);
            }
            int32_t tok = d[(int64_t)b * N + i];
            if (tok < 0 || tok >= V) err = 1;
        }
        if (err) {
            mark_error(o, b, width);
            free(lse_q);
            free(lse_p);
            continue;
        }
        /* every position is tested (the decisions past the first rejection are
         * reported but do not change the outcome) */
        int k = N;
        for (int i = 0; i < N; ++i) {
            const void* qr = row_ptr(zq, dtype, q_seq_stride, q_row_stride, b, i);
            const void* pr = row_ptr(zp, dtype, p_seq_stride, p_row_stride, b, i);
            int32_t tok = d[(int64_t)b * N + i];
            double u;
            if (u_in)
                u = u_in[(int64_t)b * (2 * N + 1) + i];
            else
                orc_uniforms(seed, round, (uint32_t)b, (uint32_t)(i + 1), &u, NULL);
            double qt, pt, r;
            int a = accept_token(logit_at(qr, dtype, tok) / T, lse_q[i], logit_at(pr, dtype, tok) / T, lse_p[i], u,
                                 &qt, &pt, &r);
            int64_t at = (int64_t)b * N + i;
            OUT_I32(o, accept, at, a);
            OUT_F64(o, q_tok, at, qt);
            OUT_F64(o, p_tok, at, pt);
            OUT_F64(o, ratio, at, r);
            OUT_F64(o, u_acc, at, u);
            if (!a && k == N) k = i; /* first rejection at position i+1 */
        }
        /* sampling slot k+1: residual of rows k, or the bonus from q row N */
        double us;
        if (u_in)
            us = u_in[(int64_t)b * (2 * N + 1) + N + k];
        else
            orc_uniforms(seed, round, (uint32_t)b, (uint32_t)(k + 1), NULL, &us);
        int tok;
        if (k < N) {
            const void* qr = row_ptr(zq, dtype, q_seq_stride, q_row_stride, b, k);
            const void* pr = row_ptr(zp, dtype, p_seq_stride, p_row_stride, b, k);
            tok = sample_at(o, b, qr, lse_q[k], 1, pr, lse_p[k], dtype, V, T, us);
        } else {
            const void* qr = row_ptr(zq, dtype, q_seq_stride, q_row_stride, b, N);
            tok = sample_at(o, b, qr, 0.0, 0, NULL, 0.0, dtype, V, T, us);
        }
        if (tok < 0) {
            mark_error(o, b, width);
            free(lse_q);
            free(lse_p);
            continue;
        }
        for (int i = 0; i < width; ++i) {
            int32_t v = -1;
            if (i < k) v = d[(int64_t)b * N + i];
            else if (i == k) v = tok;
            OUT_I32(o, tokens, (int64_t)b * width + i, v);
        }
        OUT_I32(o, num_accepted, b, k);
        OUT_I32(o, stop_node, b, k);
        free(lse_q);
        free(lse_p);
    }
    return 0;
}

/* ------------------------------------------------------------------------- */
/* Tree verify ([ZH] section 3 "why a tree, and how one pass verifies it":   */
/* the tree is flattened, every node numbered, a node sees only itself and   */
/* its ancestors; [ZH] section 4 "eagle_round" step 4 walks the tree from    */
/* the root; [PT] O Conceito / EAGLE-2).  Walk reading R5.                    */
/*                                                                           */
/* zq, zp: [B, T+1, V] rows per node (node 0 = root; leaf p rows never read).*/
/* node_tokens: [B, T+1] (entry 0 ignored).  parents: [T+1] when shared,     */
/* else [B, T+1]; parents[n] must lie in [0, n) for n >= 1.                  */
/* u_in (optional) gives per sequence T + max_depth + 1 uniforms: the accept  */
/* uniforms of nodes 1..T, then the sampling uniforms of slots              */
/* 1..max_depth+1.  walk: 0 = reading R5, 1 = reading R5b.                   */
/* ------------------------------------------------------------------------- */
int orc_verify_tree(const void* zq, int64_t q_seq_stride, int64_t q_row_stride, const void* zp,
                    int64_t p_seq_stride, int64_t p_row_stride, int dtype, const int32_t* node_tokens,
                    const int32_t* parents, int parents_shared, int B, int T, int V, int max_depth, int walk,
                    uint64_t seed, uint64_t round, double temp, const double* u_in, int b_begin, int b_end,
                    int nthreads, orc_out* o)
{
    if (B < 0 || T < 0 || V <= 0 || max_depth < 0 || !(temp > 0.0) || b_begin < 0 || b_end > B || !o ||
        !o->tokens || !o->num_accepted || (walk != 0 && walk != 1))
        return 1;
    const int nn = T + 1;
    const int width = max_depth + 1;
    const int nu = T + max_depth + 1;
#ifdef _OPENMP
    if (nthreads < 1) nthreads = 1;
#pragma omp parallel for schedule(dynamic, 1) num_threads(nthreads)
#endif
    for (int b = b_begin; b < b_end; ++b) {
        const int32_t* par = parents_shared ? parents : parents + (int64_t)b * nn;
        const int32_t* tok = node_tokens + (int64_t)b * nn;
        int err = 0;
        int* has_child = (int*)calloc((size_t)nn, sizeof(int));
        double* lse_q = (double*)malloc(sizeof(double) * (size_t)nn);
        double* lse_p = (double*)malloc(sizeof(double) * (size_t)nn);
        int* acc = (int*)calloc((size_t)nn, sizeof(int));
        for (int n = 0; n < nn; ++n) {
            lse_q[n] = NAN;
            lse_p[n] = NAN;
        }
        for (int n = 1; n < nn; ++n) {
            if (par[n] < 0 || par[n] >= n) err = 1;
            else has_child[par[n]] = 1;
            if (tok[n] < 0 || tok[n] >= V) err = 1;
        }
        /* statistics of q and p at every node that has children */
        for (int n = 0; n < nn && !err; ++n) {
            if (!has_child[n]) continue;
            const void* qr = row_ptr(zq, dtype, q_seq_stride, q_row_stride, b, n);
            const void* pr = row_ptr(zp, dtype, p_seq_stride, p_row_stride, b, n);
            if (orc_row_lse(qr, dtype, V, temp, NULL, &lse_q[n]) != 0) err = 1;
            if (!err && orc_row_lse(pr, dtype, V, temp, NULL, &lse_p[n]) != 0) err = 1;
        }
        if (!err) {
            for (int n = 0; n < nn; ++n) {
                OUT_F64(o, lse_q, (int64_t)b * nn + n, lse_q[n]);
                OUT_F64(o, lse_p, (int64_t)b * nn + n, lse_p[n]);
            }
        }
        if (err) {
            mark_error(o, b, width);
            free(has_child); free(lse_q); free(lse_p); free(acc);
            continue;
        }
        /* every node is tested against the distributions of its parent */
        OUT_I32(o, accept, (int64_t)b * nn, 1);
        OUT_F64(o, q_tok, (int64_t)b * nn, 0.0);
        OUT_F64(o, p_tok, (int64_t)b * nn, 0.0);
        OUT_F64(o, ratio, (int64_t)b * nn, 0.0);
        OUT_F64(o, u_acc, (int64_t)b * nn, 0.0);
        acc[0] = 1;
        for (int n = 1; n < nn; ++n) {
            int pa = par[n];
            const void* qr = row_ptr(zq, dtype, q_seq_stride, q_row_stride, b, pa);
            const void* pr = row_ptr(zp, dtype, p_seq_stride, p_row_stride, b, pa);
            double u;
            if (u_in)
                u = u_in[(int64_t)b * nu + (n - 1)];
            else
                orc_uniforms(seed, round, (uint32_t)b, (uint32_t)n, &u, NULL);
            double qt, pt, r;
            acc[n] = accept_token(logit_at(qr, dtype, tok[n]) / temp, lse_q[pa], logit_at(pr, dtype, tok[n]) / temp,
                                  lse_p[pa], u, &qt, &pt, &r);
            int64_t at = (int64_t)b * nn + n;
            OUT_I32(o, accept, at, acc[n]);
            OUT_F64(o, q_tok, at, qt);
            OUT_F64(o, p_tok, at, pt);
            OUT_F64(o, ratio, at, r);
            OUT_F64(o, u_acc, at, u);
        }
        /* the walk (R5, or R5b when walk = 1) */
        int* path = (int*)malloc(sizeof(int) * (size_t)(width > 0 ? width : 1));
        int depth = 0, cur = 0;
        path[0] = 0;
        int residual = 0;
        for (;;) {
            if (!has_child[cur]) break; /* leaf: bonus from q at cur */
            int next = -1;
            for (int n = cur + 1; n < nn; ++n) {
                if (par[n] != cur) continue;
                if (walk == 1) {        /* R5b: the best child decides alone */
                    if (acc[n]) next = n;
                    break;
                }
                if (acc[n]) {           /* R5: the first accepted child */
                    next = n;
                    break;
                }
            }
            if (next < 0) {
                residual = 1;
                break;
            }
            if (depth + 1 > max_depth) {
                err = 1;
                break;
            }
            path[++depth] = next;
            cur = next;
        }
        if (err) {
            mark_error(o, b, width);
            free(path); free(has_child); free(lse_q); free(lse_p); free(acc);
            continue;
        }
        double us;
        if (u_in)
            us = u_in[(int64_t)b * nu + T + depth];
        else
            orc_uniforms(seed, round, (uint32_t)b, (uint32_t)(depth + 1), NULL, &us);
        const void* qr = row_ptr(zq, dtype, q_seq_stride, q_row_stride, b, cur);
        int sampled;
        if (residual) {
            const void* pr = row_ptr(zp, dtype, p_seq_stride, p_row_stride, b, cur);
            sampled = sample_at(o, b, qr, lse_q[cur], 1, pr, lse_p[cur], dtype, V, temp, us);
        } else {
            sampled = sample_at(o, b, qr, 0.0, 0, NULL, 0.0, dtype, V, temp, us);
        }
        if (sampled < 0) {
            mark_error(o, b, width);
            free(path); free(has_child); free(lse_q); free(lse_p); free(acc);
            continue;
        }
        for (int i = 0; i < width; ++i) {
            int32_t v = -1, pn = -1;
            if (i < depth) v = tok[path[i + 1]];
            else if (i == depth) v = sampled;
            if (i <= depth) pn = path[i];
            OUT_I32(o, tokens, (int64_t)b * width + i, v);
            OUT_I32(o, path_nodes, (int64_t)b * width + i, pn);
        }
        OUT_I32(o, num_accepted, b, depth);
        OUT_I32(o, stop_node, b, cur);
        free(path); free(has_child); free(lse_q); free(lse_p); free(acc);
    }
    return 0;
}

/* ------------------------------------------------------------------------- */
/* KV rollback / compaction ([PT] Implementando, Passo 4 and "Reversao de KV */
/* cache": a logical length that is truncated on rejection; [ZH] section 3: */
/* after acceptance the KV rows of the accepted path are copied together and */
/* the other branches dropped).  L0 = kv_len_in[b] is the KV row of node 0   */
/* (the pending token); node n was written at row L0 + n by the verify pass. */
/* Accepting k drafts keeps rows L0 .. L0+k, so kv_len = L0 + k + 1 and     */
/* src_rows[i] = L0 + path[i] (identity for a chain, path_nodes == NULL).    */
/* The gather (kv != NULL) moves row L0+path[i] to row L0+i for every plane, */
/* reading every source row before writing any destination row.  A sequence */
/* with num_accepted < 0 keeps kv_len_in and gets -1 rows.                   */
/* Strides are in bytes.                                                     */
/* ------------------------------------------------------------------------- */
int orc_kv_compact(const int32_t* path_nodes, const int32_t* num_accepted, const int32_t* kv_len_in, int B,
                   int max_depth, int32_t* out_src_rows, int32_t* out_kv_len, void* kv, int64_t seq_stride,
                   int64_t row_stride, int row_bytes, int n_planes, int64_t plane_stride)
{
    if (B < 0 || max_depth < 0) return 1;
    const int width = max_depth + 1;
    for (int b = 0; b < B; ++b) {
        int k = num_accepted[b];
        int L0 = kv_len_in[b];
        if (k < 0 || k > max_depth) {
            for (int i = 0; i < width; ++i) out_src_rows[(int64_t)b * width + i] = -1;
            out_kv_len[b] = L0;
            continue;
        }
        for (int i = 0; i < width; ++i) {
            int32_t v = -1;
            if (i <= k) v = L0 + (path_nodes ? path_nodes[(int64_t)b * width + i] : i);
            out_src_rows[(int64_t)b * width + i] = v;
        }
        out_kv_len[b] = L0 + k + 1;
        if (!kv || k == 0) continue;
        unsigned char* staging = (unsigned char*)malloc((size_t)(k + 1) * (size_t)row_bytes);
        for (int pl = 0; pl < n_planes; ++pl) {
            unsigned char* seqbase = (unsigned char*)kv + pl * plane_stride + (int64_t)b * seq_stride;
            for (int i = 0; i <= k; ++i)
                memcpy(staging + (size_t)i * row_bytes,
                       seqbase + (int64_t)out_src_rows[(int64_t)b * width + i] * row_stride, (size_t)row_bytes);
            for (int i = 0; i <= k; ++i)
                memcpy(seqbase + (int64_t)(L0 + i) * row_stride, staging + (size_t)i * row_bytes,
                       (size_t)row_bytes);
        }
        free(staging);
    }
    return 0;
}

/* ------------------------------------------------------------------------- */
/* Tree attention mask and position ids ("投机解码与 EAGLE", section 3: the     */
/* flattened tree is verified in one pass in which each node sees only itself */
/* and its ancestors).  Row n of sequence b has bit j set iff j is n or an    */
/* ancestor of n, found by following parent links from n to the root;         */
/* positions[n] = L0 + depth(n).  Parents breaking parent[0] = -1,            */
/* 0 <= parent[n] < n zero the sequence's mask and set its positions to -1.   */
/* mask is [B][T+1][W] 64-bit words, W = ceil((T+1)/64), bit j of the row is  */
/* bit (j % 64) of word j / 64.                                               */
/* ------------------------------------------------------------------------- */
int orc_tree_mask(const int32_t* parents, int parents_shared, const int32_t* kv_len_in, int B, int T,
                  uint64_t* mask, int32_t* positions)
{
    if (B < 0 || T < 0) return 1;
    const int nn = T + 1, W = (nn + 63) / 64;
    for (int b = 0; b < B; ++b) {
        const int32_t* par = parents_shared ? parents : parents + (int64_t)b * nn;
        int ok = par[0] == -1;
        for (int n = 1; n < nn; ++n)
            if (par[n] < 0 || par[n] >= n) ok = 0;
        const int L0 = kv_len_in ? kv_len_in[b] : 0;
        for (int n = 0; n < nn; ++n) {
            uint64_t* row = mask + ((int64_t)b * nn + n) * W;
            for (int w = 0; w < W; ++w) row[w] = 0;
            if (!ok) {
                positions[(int64_t)b * nn + n] = -1;
                continue;
            }
            int depth = 0;
            for (int j = n;; j = par[j]) {
                row[j / 64] |= (uint64_t)1 << (j % 64);
                if (j == 0) break;
                ++depth;
            }
            positions[(int64_t)b * nn + n] = L0 + depth;
        }
    }
    return 0;
}

/* ------------------------------------------------------------------------- */
/* EAGLE-2 dynamic draft tree ("投机解码与 EAGLE", section 4, eagle_round step */
/* 2: every frontier node adds its top-k draft tokens as children with score  */
/* parent score * p(token); the dynamic tree (section 5, EAGLE-2) picks the   */
/* globally best nodes to expand and keeps the best `budget` overall).        */
/*                                                                           */
/* rows [B][n_exp][V] (strides in elements): the draft logits of the expanded */
/* nodes -- row 0 the root's, then for level l = 1..depth-1 the `topk` rows   */
/* of level l's frontier in rank order (row 1 + (l-1)*topk + r).              */
/* Readings: scores are kept as log-scores (sums of ln p, the logarithm of    */
/* the pages' product: same order, no underflow); p = softmax(logits / T);    */
/* a row's top-k is taken by (logit desc, token asc); the frontier of level   */
/* l is the top-k of level l's candidates and the kept set the top-budget of */
/* all candidates, both by (score desc, creation order asc), creation order  */
/* being level, then frontier rank, then token rank; the kept nodes are      */
/* numbered 1..budget by (level asc, score desc, creation order asc).  The    */
/* kept set is ancestor-closed: a child's score never exceeds its parent's   */
/* and the parent was created first.                                         */
/* Outputs [B][budget+1]: parents (node 0: -1), tokens (node 0: 0), depth,   */
/* log-score (node 0: 0); frontier_out (optional) [B][depth-1][topk]: the    */
/* candidate ids of each level's frontier.  A sequence with NaN or +inf in   */
/* an expanded row, or a row of -inf only, gets -1 in every output slot.    */
/* Returns 1 on bad sizes.                                                  */
/* ------------------------------------------------------------------------- */
typedef struct {
    double score;
    int id;
} scored_id;

static int by_score_then_id(const void* a, const void* b)
{
    const scored_id* x = (const scored_id*)a;
    const scored_id* y = (const scored_id*)b;
    if (x->score > y->score) return -1;
    if (x->score < y->score) return 1;
    return (x->id > y->id) - (x->id < y->id);
}

int orc_tree_build(const void* rows, int64_t seq_stride, int64_t row_stride, int dtype, int B, int V, int depth,
                   int topk, int budget, double T, int32_t* out_parents, int32_t* out_tokens, int32_t* out_depth,
                   double* out_score, int32_t* frontier_out)
{
    if (B < 0 || V < 1 || depth < 1 || topk < 1 || topk > V || budget < 1 || !(T > 0.0)) return 1;
    const int n_cand = topk + (depth - 1) * topk * topk;
    if (budget > n_cand) return 1;
    const int nn = budget + 1;
    int* c_tok = (int*)malloc(sizeof(int) * n_cand);
    int* c_par = (int*)malloc(sizeof(int) * n_cand);
    int* c_lev = (int*)malloc(sizeof(int) * n_cand);
    double* c_score = (double*)malloc(sizeof(double) * n_cand);
    scored_id* order = (scored_id*)malloc(sizeof(scored_id) * n_cand);
    int* node_of = (int*)malloc(sizeof(int) * n_cand);
    int* top_tok = (int*)malloc(sizeof(int) * topk);
    double* top_val = (double*)malloc(sizeof(double) * topk);
    int* f_ids = (int*)malloc(sizeof(int) * topk);
    double* f_score = (double*)malloc(sizeof(double) * topk);
    for (int b = 0; b < B; ++b) {
        int n = 0, F = 1, bad = 0;
        f_ids[0] = -1;
        f_score[0] = 0.0;
        for (int level = 1; level <= depth; ++level) {
            const int first = n;
            for (int f = 0; f < F; ++f) {
                const int slot = level == 1 ? 0 : 1 + (level - 2) * topk + f;
                const void* row = row_ptr(rows, dtype, seq_stride, row_stride, b, slot);
                double m, lse;
                if (orc_row_lse(row, dtype, V, T, &m, &lse)) bad = 1;
                /* top-k by (logit desc, token asc): one pass over the row
                   keeping a sorted list; a later token displaces only a
                   strictly smaller logit */
                int cnt = 0;
                for (int t = 0; t < V; ++t) {
                    const double v = logit_at(row, dtype, t);
                    if (cnt == topk && !(v > top_val[topk - 1])) continue;
                    int pos = cnt < topk ? cnt++ : topk - 1;
                    while (pos > 0 && top_val[pos - 1] < v) {
                        top_val[pos] = top_val[pos - 1];
                        top_tok[pos] = top_tok[pos - 1];
                        --pos;
                    }
                    top_val[pos] = v;
                    top_tok[pos] = t;
                }
                for (int r = 0; r < topk; ++r) {
                    c_tok[n] = top_tok[r];
                    c_par[n] = f_ids[f];
                    c_lev[n] = level;
                    c_score[n] = f_score[f] + (top_val[r] / T - lse);
                    ++n;
                }
            }
            if (level < depth) {
                const int cnt = n - first;
                for (int i = 0; i < cnt; ++i) {
                    order[i].score = c_score[first + i];
                    order[i].id = first + i;
                }
                qsort(order, (size_t)cnt, sizeof(scored_id), by_score_then_id);
                F = topk;
                for (int r = 0; r < topk; ++r) {
                    f_ids[r] = order[r].id;
                    f_score[r] = order[r].score;
                    if (frontier_out) frontier_out[((int64_t)b * (depth - 1) + (level - 1)) * topk + r] = order[r].id;
                }
            }
        }
        /* the kept set: top-budget of all candidates */
        for (int i = 0; i < n; ++i) {
            order[i].score = c_score[i];
            order[i].id = i;
            node_of[i] = -1;
        }
        qsort(order, (size_t)n, sizeof(scored_id), by_score_then_id);
        /* number the kept nodes by (level asc, score desc, id asc): a stable
           pass per level over the kept set in score order */
        int next = 1;
        for (int level = 1; level <= depth; ++level)
            for (int i = 0; i < budget; ++i)
                if (c_lev[order[i].id] == level) node_of[order[i].id] = next++;
        int32_t* P = out_parents + (int64_t)b * nn;
        int32_t* K = out_tokens + (int64_t)b * nn;
        int32_t* D = out_depth + (int64_t)b * nn;
        double* S = out_score + (int64_t)b * nn;
        if (bad) { /* NaN or +inf in an expanded row, or a row of -inf only */
            for (int i = 0; i < nn; ++i) {
                P[i] = K[i] = D[i] = -1;
                S[i] = 0.0;
            }
            continue;
        }
        P[0] = -1;
        K[0] = 0;
        D[0] = 0;
        S[0] = 0.0;
        for (int i = 0; i < budget; ++i) {
            const int c = order[i].id;
            const int node = node_of[c];
            P[node] = c_par[c] < 0 ? 0 : node_of[c_par[c]];
            K[node] = c_tok[c];
            D[node] = c_lev[c];
            S[node] = c_score[c];
        }
    }
    free(c_tok);
    free(c_par);
    free(c_lev);
    free(c_score);
    free(order);
    free(node_of);
    free(top_tok);
    free(top_val);
    free(f_ids);
    free(f_score);
    return 0;
}

/* ------------------------------------------------------------------------- */
/* Primitives exposed for the pins.                                           */
/* ------------------------------------------------------------------------- */

/* min(1, q(d)/p(d)) of one (q row, p row, token) triple, or 1 when p(d) = 0. */
double orc_accept_prob(const void* qrow, const void* prow, int dtype, int V, double T, int d)
{
    double lq, lp;
    if (orc_row_lse(qrow, dtype, V, T, NULL, &lq) || orc_row_lse(prow, dtype, V, T, NULL, &lp)) return NAN;
    double qt, pt, r;
    /* u = 0 is accepted whenever the threshold is positive; the threshold
     * itself is what the pins need */
    accept_token(logit_at(qrow, dtype, d) / T, lq, logit_at(prow, dtype, d) / T, lp, 0.0, &qt, &pt, &r);
    return r < 1.0 ? r : 1.0;
}

/* The normalised residual distribution of (q row, p row); returns its kind. */
int orc_residual_probs(const void* qrow, const void* prow, int dtype, int V, double T, double* out)
{
    double lq, lp, resid;
    if (orc_row_lse(qrow, dtype, V, T, NULL, &lq) || orc_row_lse(prow, dtype, V, T, NULL, &lp)) return KIND_ERROR;
    int kind = residual_weights(qrow, lq, prow, lp, dtype, V, T, out, &resid);
    double s = 0.0;
    for (int t = 0; t < V; ++t) s += out[t];
    for (int t = 0; t < V; ++t) out[t] /= s;
    return kind;
}

/* The token the inverse CDF picks from unnormalised weights w for uniform u. */
int orc_inverse_cdf(const double* w, int V, double u)
{
    double W, target, lo, hi;
    return inverse_cdf(w, V, u, &W, &target, &lo, &hi);
}

int orc_num_threads_available(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}
