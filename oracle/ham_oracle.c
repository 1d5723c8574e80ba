/*
 * ham_oracle.c -- plain, slow, token-serial CPU oracle of one HAM layer.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path may link, load or call
 * this file; only the tests, the smoke check and the benchmark's CPU-baseline leg
 * use it.  It shares no code, header or constant with the HIP library.
 *
 * Source: "Hybrid Associative Memories" (Lufkin, Figliolia, Millidge,
 * Krishnamurthy; arXiv 2603.22325, full-text page), cited below as [HAM].
 *
 * Everything is double precision.  The caller passes the exact input values
 * (bf16 inputs are widened exactly).  Each (b,h) head is independent and is
 * processed strictly in token order; the caller may split the head range over
 * threads.  No blocking, chunking or reordering beyond the definitions.
 *
 * Per head, with the state S stored d_k x d_v ([HAM] App. A.1, "RNN Memory"):
 *
 *   alpha_t = exp(g_t)                                  (g_t <= 0 is the log decay)
 *   p_t     = S_{t-1}^T k_t                             prediction of v_t
 *             ([HAM] App. A.1 "Router Implementations", fit-error router)
 *   e_t     = 1 - cos(p_t, v_t)   (cos := 0 if either vector is zero)
 *             ([HAM] §2 "Prediction Error as Routing Metric")
 *   routed  = float(e_t) > tau_{t,h}   (strict; NaN never routes).  The threshold
 *             is given per token and head: a constant per head, or a schedule along
 *             the sequence ([HAM] §6: the growth of the KV cache can follow a target
 *             schedule along the sequence, set at test time).
 *             With a learned input router the score is instead the caller's
 *             e_t = router_score_t (sigma(W_r x_t) or sigma(MLP(x_t)), computed
 *             outside the layer; [HAM] App. A.1 "Router Implementations", input
 *             router, and "Forward Pass": scale s = 1 for learned routers); the
 *             RNN still reads every token.
 *   S_t     = alpha_t (I - beta_t k_t k_t^T) S_{t-1} + beta_t k_t v_t^T
 *             ([HAM] §2 DeltaNet update, one gradient step on 1/2|S k - v|^2,
 *              with the gated-DeltaNet decay on the whole old state, App. A.1)
 *   o_rnn_t = S_t^T q_t                                 (post-update readout, [HAM] §2
 *                                                       linear-attention equation)
 *   Block-contiguous routing ([HAM] §7 proposes sending contiguous blocks of tokens
 *   to the KV cache instead of single tokens; the pages give no rule, so this
 *   reading is ours): with route_block = n > 1 the positions are cut into aligned
 *   blocks of n tokens; at a block's last token the block's mean score,
 *   float(sum of its e / n) compared in fp32, decides for the whole block against
 *   tau at that last token, and the n tokens are then appended together.  Until
 *   then they are not in the cache, so a query sees a routed block from the
 *   block's last token on (causal: the decision reads no later token).  n = 1 is
 *   the per-token rule.  A call starts at a block boundary; a block left open at
 *   the end of the call stays unrouted.
 *   if routed: append (k^a_t, v^a_t, position) to this head's cache
 *   (with a rotary base b > 0 the attention-path query and key are rotated at
 *    their original positions first: RoPE, [HAM] §4 model setup (rotary base
 *    500000 on the attention path's inputs), citing Su et al.'s RoFormer: consecutive
 *    pairs (x_2i, x_2i+1) turned by the angle position * b^(-2i/d_k))
 *   o_kv_t  = softmax over the cached keys, scale * q^a_t . k_c, of the cached
 *             values; 0 when no cached key is visible     ([HAM] §2 KV-memory
 *             equation; causality by original position, App. A.1 "FlexAttention
 *             and Block Masks")
 *             Same-document masking (same passage): in a packed sequence each
 *             document is a contiguous range of positions, and doc_start[b,t] is
 *             the position where token t's document begins.  A cached key is
 *             visible to the query only when its position is >= doc_start (it
 *             belongs to the same document; documents may span calls).  Only the
 *             attention is masked: the RNN and the routing read every token.
 *   o_t     = gr_t * rms(o_rnn_t) + gk_t * rms(o_kv_t),  rms(x) = x / sqrt(mean(x^2)+eps)
 *             ([HAM] §2 headwise norm and gated sum; App. A.1 headwise gating)
 *
 * Parity pins for every function here live in tests/test_oracle_pins.py.
 */
#include <math.h>
#include <stddef.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* RoPE ([HAM] §4 model setup: rotary base 500000 on the attention inputs; RoFormer):
 * y_2i = x_2i cos(a_i) - x_2i+1 sin(a_i), y_2i+1 = x_2i sin(a_i) + x_2i+1 cos(a_i),
 * a_i = pos * base^(-2i/d).  y may not alias x. */
static void rope_rotate(const double *x, double *y, int d, double pos, double base)
{
    for (int i = 0; i < d / 2; ++i) {
        const double a = pos * pow(base, -2.0 * i / d);
        const double c = cos(a), s = sin(a);
        y[2 * i] = x[2 * i] * c - x[2 * i + 1] * s;
        y[2 * i + 1] = x[2 * i] * s + x[2 * i + 1] * c;
    }
}

/* cosine of two vectors; 0 when either has zero norm.  [HAM] §2 routing score. */
static double cosine(const double *a, const double *b, int n)
{
    double ab = 0.0, aa = 0.0, bb = 0.0;
    for (int i = 0; i < n; ++i) {
        ab += a[i] * b[i];
        aa += a[i] * a[i];
        bb += b[i] * b[i];
    }
    if (aa == 0.0 || bb == 0.0)
        return 0.0;
    double c = ab / (sqrt(aa) * sqrt(bb));
    if (c > 1.0) c = 1.0;
    if (c < -1.0) c = -1.0;
    return c;
}

/* x / sqrt(mean(x^2) + eps), written to y.  [HAM] §2 Norm_h of each readout. */
static void rms_normalize(const double *x, double *y, int n, double eps)
{
    double ss = 0.0;
    for (int i = 0; i < n; ++i)
        ss += x[i] * x[i];
    double inv = 1.0 / sqrt(ss / (double)n + eps);
    for (int i = 0; i < n; ++i)
        y[i] = x[i] * inv;
}

/*
 * One HAM layer over RNN heads [head_begin, head_end) of the flattened B x H grid
 * (head index = b*H + h), for T new tokens.
 *
 * Attention (KV) heads: Hk of them (0 = H) with key/value sizes dkk, dvk (0 = dk,
 * dv); Hk = r*H.  KV head j = r*h + i follows the routing of RNN head h and holds
 * its own cache; the values of KV heads r*h .. r*h+r-1 lie side by side over the
 * dv = r*dvk output columns of RNN head h ([HAM] §4 model setup: twice the RNN
 * heads at half their size, the value size chosen to match the RNN's output;
 * App. E Tab. E.1).  Each side is RMS-normalised per head of its own size and
 * gated per head (gate_kv per KV head) before the sum.
 *
 * Layouts (row-major): RNN token tensors [B,T,H,d]; attention-path tensors
 * [B,T,Hk,dkk|dvk]; per-token scalars [B,T,H] (gate_kv [B,T,Hk]); state S
 * [B,H,dk,dv] (read as the entering state, overwritten with S_T); cache Kc
 * [B,Hk,cap,dkk], Vc [B,Hk,cap,dvk], pos [B,Hk,cap], count [B,Hk] (read as the
 * entering cache, extended in place); o_kv [B,T,Hk,dvk]; o, o_rnn [B,T,H,dv].
 * t0[b] is the absolute position of token 0 of sequence b.  qa/ka/va: separate
 * attention-path inputs, or NULL to share q/k/v (only with the RNN's geometry;
 * [HAM] §2 implementation details: shared projections).  gate_rnn/gate_kv: NULL
 * means 1.  mask_override: NULL, or a [B,T,H] array of 0/1 that replaces the
 * threshold decision (the score e is still computed).  router_score: NULL, or a
 * [B,T,H] fp32 array of routing scores that replaces the fit-error score (e is
 * then a copy of it).  emit: NULL, or a [B,T,H] 0/1 array; where it is 0 the
 * attention readout and the mix of that token are skipped (o_kv and o stay as
 * they were) -- this only saves time when a few sampled tokens are checked.
 * rope_base: 0 for none, else the rotary base applied to the attention-path
 * query and key at their absolute positions (the cache then holds rotated keys).
 * route_block: 0 or 1 for per-token routing, else the block size of
 * block-contiguous routing (every t0[b] a multiple of it).  With mask_override,
 * a block's decision is the override at its last token.
 * Outputs e, routed, o_rnn, o_kv, o may each be NULL.
 *
 * Returns 0, -1 if a t0[b] is not a multiple of route_block or the head geometry
 * is inconsistent, or -3 if a routed token finds the cache full (the head stops).
 */
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
                       int head_begin, int head_end)
{
    if (Hk <= 0) Hk = H;
    if (dkk <= 0) dkk = dk;
    if (dvk <= 0) dvk = dv;
    const int r = Hk / H;
    const int own = (Hk != H || dkk != dk || dvk != dv);
    if (Hk % H != 0 || r * dvk != dv || (own && !(qa && ka && va)))
        return -1;
    const double *qA = qa ? qa : q;
    const double *kA = ka ? ka : k;
    const double *vA = va ? va : v;
    double *p = (double *)malloc(sizeof(double) * (size_t)dv);
    double *orn = (double *)malloc(sizeof(double) * (size_t)dv);
    double *okv = (double *)malloc(sizeof(double) * (size_t)dv);    /* r heads of dvk */
    double *tmp1 = (double *)malloc(sizeof(double) * (size_t)dv);
    double *tmp2 = (double *)malloc(sizeof(double) * (size_t)dv);
    double *w = (double *)malloc(sizeof(double) * (size_t)(cap > 0 ? cap : 1));
    double *qrot = (double *)malloc(sizeof(double) * (size_t)dkk);
    int64_t *n = (int64_t *)malloc(sizeof(int64_t) * (size_t)r);
    int status = 0;
    const int nb = route_block > 1 ? route_block : 1;
    for (int b = 0; b < B; ++b)
        if (t0[b] % nb != 0) status = -1;
    if (status) head_end = head_begin;

    for (int bh = head_begin; bh < head_end; ++bh) {
        const int b = bh / H, h = bh % H;
        double *Sh = S + (size_t)bh * dk * dv;
        for (int i = 0; i < r; ++i)
            n[i] = count[(size_t)b * Hk + (size_t)h * r + i];
        double bsum = 0.0;                       /* score sum of the open block */

        for (int t = 0; t < T; ++t) {
            const size_t tok = ((size_t)b * T + t) * H + h;   /* [B,T,H] index */
            const double *kt = k + tok * dk, *vt = v + tok * dv, *qt = q + tok * dk;
            const double alpha = exp(g[tok]);
            const double bt = beta[tok];

            /* prediction p = S_{t-1}^T k_t */
            for (int j = 0; j < dv; ++j) {
                double acc = 0.0;
                for (int i = 0; i < dk; ++i)
                    acc += Sh[(size_t)i * dv + j] * kt[i];
                p[j] = acc;
            }
            /* routing score and decision (decision taken in fp32, like the GPU) */
            const double et = router_score ? (double)router_score[tok] : 1.0 - cosine(p, vt, dv);
            int rt;
            const int jb = (int)((t0[b] + t) % nb);  /* place in its block */
            if (jb == 0) bsum = 0.0;
            bsum += et;
            if (jb != nb - 1)
                rt = 0;                                  /* the block is still open */
            else if (mask_override)
                rt = mask_override[tok] != 0;
            else
                rt = ((float)(bsum / nb) > tau[tok]);
            if (e) e[tok] = et;
            if (routed) {
                routed[tok] = (int8_t)rt;
                if (jb == nb - 1)                        /* the whole block shares it */
                    for (int i = 1; i < nb; ++i) routed[tok - (size_t)i * H] = (int8_t)rt;
            }

            /* gated delta update: S = alpha*S + beta*k*(v - alpha*p)^T
             * which equals alpha*(I - beta k k^T) S + beta k v^T. */
            for (int i = 0; i < dk; ++i) {
                const double bk = bt * kt[i];
                for (int j = 0; j < dv; ++j)
                    Sh[(size_t)i * dv + j] = alpha * Sh[(size_t)i * dv + j]
                                           + bk * (vt[j] - alpha * p[j]);
            }
            /* post-update readout o_rnn = S_t^T q_t */
            for (int j = 0; j < dv; ++j) {
                double acc = 0.0;
                for (int i = 0; i < dk; ++i)
                    acc += Sh[(size_t)i * dv + j] * qt[i];
                orn[j] = acc;
            }

            /* per KV head of this RNN head: append, then attend */
            for (int jj = 0; jj < r; ++jj) {
                const size_t hk = (size_t)b * Hk + (size_t)h * r + jj;   /* [B,Hk] index */
                double *Kh = Kc + hk * cap * dkk;
                double *Vh = Vc + hk * cap * dvk;
                int64_t *ph = pos + hk * cap;
                /* append the routed token (with blocks: the whole block, at its last
                 * token), ascending original position */
                if (rt) {
                    for (int ta = t - (nb - 1); ta <= t; ++ta) {
                        const size_t tk = ((size_t)b * T + ta) * Hk + (size_t)h * r + jj;
                        if (n[jj] >= cap) { status = -3; break; }
                        if (rope_base > 0.0)
                            rope_rotate(kA + tk * dkk, Kh + (size_t)n[jj] * dkk, dkk,
                                        (double)(t0[b] + ta), rope_base);
                        else
                            memcpy(Kh + (size_t)n[jj] * dkk, kA + tk * dkk, sizeof(double) * (size_t)dkk);
                        memcpy(Vh + (size_t)n[jj] * dvk, vA + tk * dvk, sizeof(double) * (size_t)dvk);
                        ph[n[jj]] = t0[b] + ta;
                        n[jj] += 1;
                    }
                    if (status) break;
                }
                if (emit && !emit[tok]) continue;
                /* softmax attention over the cached (routed) keys, all at positions <= t */
                const size_t tka = ((size_t)b * T + t) * Hk + (size_t)h * r + jj;
                const double *qat = qA + tka * dkk;
                if (rope_base > 0.0) {
                    rope_rotate(qat, qrot, dkk, (double)(t0[b] + t), rope_base);
                    qat = qrot;
                }
                double *ok = okv + (size_t)jj * dvk;
                for (int j = 0; j < dvk; ++j) ok[j] = 0.0;
                /* first position of this token's document (none: the whole cache) */
                const int64_t ds = doc_start ? doc_start[(size_t)b * T + t] : INT64_MIN;
                double m = -INFINITY;
                int64_t nvis = 0;
                for (int64_t c = 0; c < n[jj]; ++c) {
                    if (ph[c] < ds) { w[c] = -INFINITY; continue; }   /* another document */
                    double sc = 0.0;
                    for (int i = 0; i < dkk; ++i)
                        sc += qat[i] * Kh[(size_t)c * dkk + i];
                    w[c] = scale * sc;
                    if (w[c] > m) m = w[c];
                    nvis += 1;
                }
                if (nvis > 0) {
                    double den = 0.0;
                    for (int64_t c = 0; c < n[jj]; ++c) {
                        w[c] = (w[c] == -INFINITY) ? 0.0 : exp(w[c] - m);
                        den += w[c];
                    }
                    for (int64_t c = 0; c < n[jj]; ++c) {
                        const double wc = w[c] / den;
                        for (int j = 0; j < dvk; ++j)
                            ok[j] += wc * Vh[(size_t)c * dvk + j];
                    }
                }
            }
            if (status) break;

            if (emit && !emit[tok]) {
                if (o_rnn) memcpy(o_rnn + tok * dv, orn, sizeof(double) * (size_t)dv);
                continue;
            }
            /* headwise RMS norms (each side per head of its own size) and the gates */
            const double gr = gate_rnn ? gate_rnn[tok] : 1.0;
            rms_normalize(orn, tmp1, dv, eps);
            for (int jj = 0; jj < r; ++jj)
                rms_normalize(okv + (size_t)jj * dvk, tmp2 + (size_t)jj * dvk, dvk, eps);
            for (int c = 0; c < dv; ++c) {
                const int jj = c / dvk;
                const size_t tka = ((size_t)b * T + t) * Hk + (size_t)h * r + jj;
                const double gk = gate_kv ? gate_kv[tka] : 1.0;
                if (o_rnn) o_rnn[tok * dv + c] = orn[c];
                if (o_kv) o_kv[tka * dvk + (c - jj * dvk)] = okv[c];
                if (o) o[tok * dv + c] = gr * tmp1[c] + gk * tmp2[c];
            }
        }
        for (int i = 0; i < r; ++i)
            count[(size_t)b * Hk + (size_t)h * r + i] = n[i];
        if (status) break;
    }
    free(p); free(orn); free(okv); free(tmp1); free(tmp2); free(w); free(qrot); free(n);
    return status;
}
