/*
 * Driver of oracle/ham_oracle.c for the host sanitizer build (AddressSanitizer and
 * UndefinedBehaviorSanitizer).  Runs ham_oracle_forward over small seeded inputs in
 * every configuration it takes -- plain, twice the KV heads with their own inputs,
 * RoPE with same-document masks and gates, block routing with a learned-router
 * score, a routing override with sampled emission, a partial head range, a cache
 * continued from an earlier call, T = 0 and T = 1 -- and over its error returns (a
 * full cache, inconsistent head geometry, a start position off the routing block).
 * Exit status 0 when every call returns its expected code and every output is
 * finite; a sanitizer report aborts the process.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

int ham_oracle_forward(int B, int T, int H, int dk, int dv, int Hk, int dkk, int dvk,
                       double scale, double eps, double rope_base, int route_block,
                       const double *q, const double *k, const double *v,
                       const double *qa, const double *ka, const double *va,
                       const double *beta, const double *g, const float *tau,
                       const double *gate_rnn, const double *gate_kv,
                       const int8_t *mask_override, const float *router_score,
                       const int8_t *emit, const int64_t *t0, const int64_t *doc_start,
                       double *S, int cap, double *Kc, double *Vc,
                       int64_t *pos, int64_t *count,
                       double *e, int8_t *routed,
                       double *o_rnn, double *o_kv, double *o,
                       int head_begin, int head_end);

static uint64_t state = 0x9E3779B97F4A7C15ull;
static double urand(void) {                 /* xorshift64*, [0, 1) */
    state ^= state >> 12; state ^= state << 25; state ^= state >> 27;
    return (double)((state * 2685821657736338717ull) >> 11) * (1.0 / 9007199254740992.0);
}
static double *dvec(size_t n, double lo, double hi) {
    double *p = (double *)malloc(sizeof(double) * (n ? n : 1));
    for (size_t i = 0; i < n; ++i) p[i] = lo + (hi - lo) * urand();
    return p;
}
static float *fvec(size_t n, double lo, double hi) {
    float *p = (float *)malloc(sizeof(float) * (n ? n : 1));
    for (size_t i = 0; i < n; ++i) p[i] = (float)(lo + (hi - lo) * urand());
    return p;
}
static int8_t *bvec(size_t n, double p1) {
    int8_t *p = (int8_t *)malloc(n ? n : 1);
    for (size_t i = 0; i < n; ++i) p[i] = urand() < p1;
    return p;
}
static int finite_all(const double *x, size_t n) {
    for (size_t i = 0; i < n; ++i)
        if (!isfinite(x[i])) return 0;
    return 1;
}

typedef struct {
    const char *name;
    int B, T, H, dk, dv, Hk, dkk, dvk;     /* Hk/dkk/dvk 0: the RNN's geometry */
    double rope;
    int block, docs, gates, learned, override, emit, own_inputs, partial, prefix, cap, t0mis;
    double tau_lo, tau_hi;
    int expect;
} Case;

static int run(const Case *c) {
    const int B = c->B, T = c->T, H = c->H, dk = c->dk, dv = c->dv;
    const int Hk = c->Hk ? c->Hk : H, dkk = c->dkk ? c->dkk : dk, dvk = c->dvk ? c->dvk : dv;
    const size_t ntok = (size_t)B * T * H, nkv = (size_t)B * T * Hk;
    const int cap = c->cap;
    double *q = dvec(ntok * dk, -1, 1), *k = dvec(ntok * dk, -1, 1), *v = dvec(ntok * dv, -1, 1);
    double *qa = c->own_inputs ? dvec(nkv * dkk, -1, 1) : NULL;
    double *ka = c->own_inputs ? dvec(nkv * dkk, -1, 1) : NULL;
    double *va = c->own_inputs ? dvec(nkv * dvk, -1, 1) : NULL;
    double *beta = dvec(ntok, 0.05, 0.9), *g = dvec(ntok, -0.3, 0.0);
    float *tau = fvec(ntok, c->tau_lo, c->tau_hi);
    double *gr = c->gates ? dvec(ntok, 0.2, 1.5) : NULL, *gk = c->gates ? dvec(nkv, 0.2, 1.5) : NULL;
    int8_t *ovr = c->override ? bvec(ntok, 0.4) : NULL;
    float *score = c->learned ? fvec(ntok, 0, 1) : NULL;
    int8_t *emit = c->emit ? bvec(ntok, 0.3) : NULL;
    int64_t *t0 = (int64_t *)malloc(sizeof(int64_t) * B);
    int64_t *docs = c->docs ? (int64_t *)malloc(sizeof(int64_t) * ((size_t)B * T + 1)) : NULL;
    double *S = dvec((size_t)B * H * dk * dv, -0.1, 0.1);
    double *Kc = dvec((size_t)B * Hk * cap * dkk, 0, 0), *Vc = dvec((size_t)B * Hk * cap * dvk, 0, 0);
    int64_t *pos = (int64_t *)calloc((size_t)B * Hk * cap + 1, sizeof(int64_t));
    int64_t *count = (int64_t *)calloc((size_t)B * Hk + 1, sizeof(int64_t));
    double *e = dvec(ntok, 0, 0), *o_rnn = dvec(ntok * dv, 0, 0), *o_kv = dvec(nkv * dvk, 0, 0);
    double *o = dvec(ntok * dv, 0, 0);
    int8_t *routed = bvec(ntok, 0);
    for (int b = 0; b < B; ++b) {
        const int blk = c->block > 1 ? c->block : 1;
        t0[b] = (int64_t)(c->prefix + blk * b) + (c->t0mis && b == B - 1 ? 1 : 0);
        for (int j = 0; j < Hk; ++j) {               /* a cache continued from an earlier call */
            const size_t bj = (size_t)b * Hk + j;
            const int n = c->prefix < cap ? c->prefix / 2 : 0;
            for (int i = 0; i < n; ++i) {
                pos[bj * cap + i] = 2 * i;
                for (int x = 0; x < dkk; ++x) Kc[(bj * cap + i) * dkk + x] = urand() - 0.5;
                for (int x = 0; x < dvk; ++x) Vc[(bj * cap + i) * dvk + x] = urand() - 0.5;
            }
            count[bj] = n;
        }
        if (docs) {
            int64_t start = 0;
            for (int t = 0; t < T; ++t) {
                const int64_t p = t0[b] + t;
                if (urand() < 0.08) start = p;
                docs[(size_t)b * T + t] = start;
            }
        }
    }
    const int hb = c->partial ? 1 : 0, he = c->partial ? B * H - 1 : B * H;
    const int rc = ham_oracle_forward(B, T, H, dk, dv, c->Hk, c->dkk, c->dvk, 1.0 / sqrt((double)dkk), 1e-6,
                                      c->rope, c->block, q, k, v, qa, ka, va, beta, g, tau, gr, gk, ovr, score,
                                      emit, t0, docs, S, cap, Kc, Vc, pos, count, e, routed, o_rnn, o_kv, o, hb, he);
    int ok = rc == c->expect;
    if (ok && rc == 0)
        ok = finite_all(o, ntok * dv) && finite_all(o_rnn, ntok * dv) && finite_all(o_kv, nkv * dvk) &&
             finite_all(S, (size_t)B * H * dk * dv);
    printf("%-28s rc %d (expected %d)%s\n", c->name, rc, c->expect, ok ? "" : "  FAILED");
    free(q); free(k); free(v); free(qa); free(ka); free(va); free(beta); free(g); free(tau); free(gr); free(gk);
    free(ovr); free(score); free(emit); free(t0); free(docs); free(S); free(Kc); free(Vc); free(pos); free(count);
    free(e); free(o_rnn); free(o_kv); free(o); free(routed);
    return ok;
}

int main(void) {
    /* name B T H dk dv Hk dkk dvk rope block docs gates learned override emit own partial prefix cap t0mis
       tau_lo tau_hi expect */
    const Case cases[] = {
        {"plain", 2, 37, 2, 8, 8, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 37, 0, 0.0, 1.0, 0},
        {"kv heads x2, own inputs", 2, 29, 2, 8, 8, 4, 8, 4, 0, 0, 0, 0, 0, 0, 0, 1, 0, 0, 29, 0, 0.0, 1.0, 0},
        {"rope, documents, gates", 2, 41, 3, 8, 6, 0, 0, 0, 10000.0, 0, 1, 1, 0, 0, 0, 0, 0, 0, 41, 0, 0.0, 1.0, 0},
        {"block routing, learned", 2, 32, 2, 8, 8, 0, 0, 0, 0, 4, 0, 0, 1, 0, 0, 0, 0, 0, 32, 0, 0.0, 1.0, 0},
        {"override, sampled emit", 1, 25, 2, 4, 8, 0, 0, 0, 0, 0, 0, 0, 0, 1, 1, 0, 0, 0, 25, 0, 0.0, 1.0, 0},
        {"partial head range", 3, 19, 2, 8, 8, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 1, 0, 19, 0, 0.0, 1.0, 0},
        {"continued cache", 2, 23, 2, 8, 8, 0, 0, 0, 500000.0, 0, 1, 0, 0, 0, 0, 0, 0, 10, 40, 0, 0.0, 1.0, 0},
        {"T = 0", 2, 0, 2, 8, 8, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 1, 0, 0.0, 1.0, 0},
        {"T = 1", 2, 1, 2, 8, 8, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 1, 0, -1.0, -1.0, 0},
        {"cache full", 1, 20, 2, 8, 8, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 3, 0, -1.0, -1.0, -3},
        {"bad kv geometry", 1, 8, 2, 8, 8, 3, 8, 8, 0, 0, 0, 0, 0, 0, 0, 1, 0, 0, 8, 0, 0.0, 1.0, -1},
        {"start off the block", 2, 16, 2, 8, 8, 0, 0, 0, 0, 4, 0, 0, 0, 0, 0, 0, 0, 0, 16, 1, 0.0, 1.0, -1},
    };
    int failures = 0;
    for (size_t i = 0; i < sizeof cases / sizeof cases[0]; ++i) failures += !run(&cases[i]);
    printf("%d failure(s)\n", failures);
    return failures == 0 ? 0 : 1;
}
