/*
 * ham.h -- C ABI of the HAM (Hybrid Associative Memory) sequence-mixer library
 * for AMD Instinct MI355X (gfx950).
 *
 * Method: "Hybrid Associative Memories" (Lufkin, Figliolia, Millidge,
 * Krishnamurthy; arXiv 2603.22325), cited as [HAM].  Per (batch b, head h):
 *
 *   gated delta-rule RNN ([HAM] §2 DeltaNet update; App. A.1 "RNN Memory"),
 *   state S in R^{dk x dv}, alpha_t = exp(g_t):
 *       S_t = alpha_t (I - beta_t k_t k_t^T) S_{t-1} + beta_t k_t v_t^T
 *       o_rnn_t = S_t^T q_t                       (post-update readout)
 *   routing score ([HAM] §2 "Prediction Error as Routing Metric"; App. A.1
 *   fit-error router):  e_t = 1 - cos(S_{t-1}^T k_t, v_t)   (cos := 0 for a
 *   zero vector), token t is routed iff e_t > tau_h (strict, in fp32); or,
 *   with ham_dims.route_block, whole blocks on their mean score.
 *   KV memory of routed tokens only ([HAM] §2 KV-memory equation; App. A.1
 *   causality by original position): o_kv_t = softmax_c(scale * q_t.Kc[c]) Vc
 *   over cached entries at original positions <= t; 0 if there are none.
 *   mix ([HAM] §2 headwise norm and gated sum; App. A.1 headwise gating):
 *       o_t = gr_t * rms(o_rnn_t) + gk_t * rms(o_kv_t),
 *       rms(x) = x / sqrt(mean(x^2) + norm_eps).
 *
 * Conventions shared by every entry point
 *   - All tensor pointers are DEVICE pointers owned by the caller; the library
 *     never allocates or frees device memory.  Scratch memory comes from the
 *     caller through (ws, ws_bytes), sized by the matching *_workspace_size().
 *   - Layouts are dense row-major: token tensors [B,T,H,d]; per-token scalars
 *     [B,T,H] fp32; state [B,H,dk,dv] fp32; KV cache [B,H,cap,d] (io dtype),
 *     pos [B,H,cap] int32, count [B,H] int32.  Pointers must be 16-byte aligned.
 *   - io_dtype selects the element type of q, k, v, the attention inputs, the
 *     cache and the outputs o / o_rnn / o_kv: HAM_F32 (float) or HAM_BF16
 *     (bfloat16 bits; stores round to nearest even).  beta, g, tau, gates, e and
 *     the state are always fp32.
 *   - dk, dv must each be 64 or 128, or dk = 256 with dv = 384 (the RNN heads of
 *     the paper's layer, run by the token-serial RNN kernel); dk_kv, dv_kv 64 or
 *     128 each, or 128 with 192 (its KV heads).  "KV heads" below
 *     are the attention heads: kv_heads of them (default H) with sizes dk_kv,
 *     dv_kv (default dk, dv); the cache, gate_kv, o_kv and the attention-path
 *     inputs are shaped by them.
 *   - `stream` is a hipStream_t (NULL = the null stream).  Every call only
 *     enqueues work; nothing blocks except ham_route_stats with rho_host != NULL.
 *   - Return codes: HAM_OK, or a negative HAM_E* code; ham_last_error() then
 *     returns a thread-local message.  Argument errors are detected on the host
 *     before anything is enqueued.
 */
#ifndef HAM_H
#define HAM_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define HAM_OK 0
#define HAM_EINVAL (-1)        /* NULL required pointer, bad size, misalignment */
#define HAM_EUNSUPPORTED (-2)  /* dk/dv not in {64,128}, unknown dtype or flag */
#define HAM_ECAPACITY (-3)     /* cap < (tokens already cached) + T */
#define HAM_EHIP (-4)          /* a HIP launch failed */
#define HAM_EWORKSPACE (-5)    /* ws NULL or smaller than the *_workspace_size() */

#define HAM_F32 0
#define HAM_BF16 1

/* flags */
#define HAM_CONTINUE 1         /* S0 / Kc / Vc / pos / count hold an earlier call's
                                  state and cache; new entries are appended */
#define HAM_FORCE_RECURRENT 2  /* run the token-serial RNN kernel even for long T */
#define HAM_EXTERNAL_SCORES 4  /* e is an input: the routing scores of a learned input
                                  router (sigma(W_r x_t) or sigma(MLP(x_t)), computed by
                                  the caller; [HAM] App. A.1 "Router Implementations",
                                  scale s = 1 in "Forward Pass") replace the RNN's
                                  prediction error; tau is in the same units.  The RNN
                                  still reads every token.  ham_forward and
                                  ham_decode_step only. */
#define HAM_OVERLAP 16         /* with HAM_EXTERNAL_SCORES (ham_forward, bf16, T > 64):
                                  the RNN does not feed the routing, so it runs on a
                                  second stream of the library's own (one per device,
                                  created on first use) beside routing, compaction and
                                  attention ([HAM] §7: with a learned router the two
                                  memories need not wait for each other); the streams
                                  join before the mix of the two readouts.  The call
                                  still only enqueues work on the caller's stream, which
                                  waits for the second one before the mix.  Calls with
                                  this flag on one device serialise their RNN work on
                                  that second stream.  Ignored without
                                  HAM_EXTERNAL_SCORES or off the chunked path. */
#define HAM_TAU_PER_TOKEN 8    /* tau holds one threshold per token and head:
                                  [B,T,H] (ham_forward, ham_route_stats) or [B,H]
                                  (ham_decode_step) instead of [H].  A schedule
                                  along the sequence steers how the KV cache grows
                                  ([HAM] §6: growth-rate control by a target
                                  schedule, set at test time). */

typedef struct {
    int B, T, H;      /* batch, new tokens per sequence, heads                   */
    int dk, dv;       /* key and value head sizes (64 or 128 each, or 256/384)   */
    int io_dtype;     /* HAM_F32 or HAM_BF16                                      */
    float scale;      /* attention logit scale, > 0 (usually 1/sqrt(dk))         */
    float norm_eps;   /* eps of the two headwise RMS norms of the mix            */
    int cap;          /* KV-cache capacity per (b,h), in tokens, 1..4194304       */
    int flags;        /* HAM_CONTINUE | HAM_FORCE_RECURRENT | HAM_EXTERNAL_SCORES
                         | HAM_TAU_PER_TOKEN | HAM_OVERLAP                        */
    int t0;           /* absolute position of token 0 (recorded in pos)          */
    float rope_base;  /* 0, or the base of a rotary position embedding (RoPE)
                         applied to the attention-path query and key at their
                         absolute positions ([HAM] §4 model setup: base 500000
                         on the attention path).  Pairs of consecutive elements
                         (x_2i, x_2i+1) turn by pos * rope_base^(-2i/dk) (RoFormer);
                         the cache then holds rotated keys.  The RNN path is not
                         rotated.  Angles are formed and reduced in double
                         precision; their (cos, sin) pairs are kept as floats in
                         a workspace table and the rotation runs in float.      */
    int route_block;  /* 0 or 1: every token is routed on its own score.  2, 4,
                         8, 16, 32 or 64: block-contiguous routing ([HAM] §7:
                         routing whole runs of adjacent tokens into the cache
                         to avoid the scattered reads of per-token routing).  The
                         positions are cut into aligned blocks of route_block
                         tokens; a block enters the cache whole when the mean
                         of its tokens' scores (summed in token order in fp32,
                         then scaled by 1/route_block) exceeds tau (taken at
                         the block's last token with HAM_TAU_PER_TOKEN), else
                         none of it does.  The decision needs the whole block,
                         so a block becomes visible to the attention from its
                         last token on: a query sees the cached blocks that end
                         at or before it.  With route_block = 1 this is the
                         per-token rule.  ham_forward and ham_route_stats take
                         whole blocks (t0 and T multiples of route_block);
                         ham_decode_step keeps the open block pending.        */
    int kv_heads;     /* 0 (= H), or the number of attention (KV) heads: H or
                         r*H with r = 2 (other multiples: HAM_EUNSUPPORTED).  The paper's layers have twice as many
                         KV heads as RNN heads, each half the RNN head's size
                         ([HAM] §4 model setup: RNN heads 256/384, KV heads
                         128/192, the value size chosen to match the RNN's
                         output; App. E Tab. E.1: h_KV = d_QK/128 = 2 h_RNN).  KV head j takes the routing of RNN
                         head j / r (its cache holds the same positions) and its
                         own attention-path q, k, v; the outputs of KV heads
                         r*h .. r*h+r-1 lie side by side over the columns of RNN
                         head h, so kv_heads * dv_kv must equal H * dv.  Each
                         side is RMS-normalised per head of its own size and
                         gated per head before the sum.                       */
    int dk_kv, dv_kv; /* 0 (= dk, dv), or the KV heads' key and value sizes (64
                         or 128 each, or 128/192).  When kv_heads != H or dk_kv != dk, the
                         attention-path inputs q_attn, k_attn, v_attn are
                         required ([B,T,kv_heads,dk_kv|dv_kv]).              */
} ham_dims;

/* Library version (major*10000 + minor*100 + patch). */
int ham_version(void);

/* Thread-local message for the last non-OK return of this thread. */
const char *ham_last_error(void);

/* Bytes of device scratch ham_forward needs for these dims (0 on bad dims). */
size_t ham_forward_workspace_size(const ham_dims *dims);

/*
 * ham_forward -- one HAM layer over T new tokens of B sequences.
 * [HAM] §2 (all four equations) and App. A.1 (router, masking, generation).
 *
 *   q, k, v            [B,T,H,dk|dv] io dtype, required: the RNN inputs.
 *   q_attn, k_attn, v_attn  attention-path inputs [B,T,kv_heads,dk_kv|dv_kv], or
 *                      NULL to share q/k/v (the paper shares the projections;
 *                      required when the KV heads' geometry differs).
 *   beta, g            [B,T,H] fp32, required: write strength and log decay
 *                      (alpha = exp(g); g must be finite).
 *   tau                [H] fp32, required: routing threshold per head in e-units
 *                      (+inf routes nothing: pure gated DeltaNet; -inf routes all);
 *                      [B,T,H] with HAM_TAU_PER_TOKEN.
 *   gate_rnn, gate_kv  [B,T,H] and [B,T,kv_heads] fp32, or NULL (= 1).
 *   doc_start          [B,T] int32 or NULL: same-document masking of a packed
 *                      batch ([HAM] App. A.1 "FlexAttention and Block Masks").
 *                      doc_start[b,t] is the absolute position where token t's
 *                      document begins; the token attends only to cached keys
 *                      at positions >= it (keys of earlier calls included, so a
 *                      document may span calls).  Only the attention is masked:
 *                      the RNN, the routing and the cache see every token.
 *                      Any values are accepted; a start after the token's own
 *                      position leaves it no key (o_kv = 0).
 *   S0                 [B,H,dk,dv] fp32 entering state, or NULL (= 0).
 *   S_out              [B,H,dk,dv] fp32, required: state after token T-1.  May
 *                      alias S0.
 *   o                  [B,T,H,dv] io dtype, required: mixed output.
 *   o_rnn, o_kv        [B,T,H,dv] and [B,T,kv_heads,dv_kv] io dtype or NULL: the
 *                      two readouts before the norms (o_kv = 0 where nothing
 *                      is visible).
 *   e                  [B,T,H] fp32 or NULL: routing scores (output).  With
 *                      HAM_EXTERNAL_SCORES it is a required input: the caller's
 *                      scores, read and not written.
 *   routed             [B,T,H] uint8 or NULL: 1 where routed.
 *   Kc, Vc, pos, count the per-(b, KV head) cache [B,kv_heads,cap,dk_kv|dv_kv],
 *                      [B,kv_heads,cap], [B,kv_heads], required.  Without HAM_CONTINUE
 *                      count is output only and entries [0,count) are written;
 *                      with it, count[b,h] (<= cap) entries already exist and
 *                      new ones are appended.  Entries are in ascending original
 *                      position; pos holds t0 + t.  Entries >= count are left
 *                      untouched.
 *   ws, ws_bytes       device scratch of ham_forward_workspace_size(dims) bytes.
 * Errors: HAM_EINVAL, HAM_EUNSUPPORTED, HAM_ECAPACITY (cap < T, or with
 * HAM_CONTINUE cap < T plus the cached tokens -- that part is checked on the
 * device: appends beyond cap are dropped and count saturates at cap),
 * HAM_EWORKSPACE, HAM_EHIP.  With route_block > 1, t0 and T must be multiples
 * of it (HAM_EINVAL).
 */
int ham_forward(const ham_dims *dims,
                const void *q, const void *k, const void *v,
                const void *q_attn, const void *k_attn, const void *v_attn,
                const float *beta, const float *g, const float *tau,
                const float *gate_rnn, const float *gate_kv,
                const int32_t *doc_start,
                const float *S0, float *S_out,
                void *o, void *o_rnn, void *o_kv,
                float *e, uint8_t *routed,
                void *Kc, void *Vc, int32_t *pos, int32_t *count,
                void *ws, size_t ws_bytes, void *stream);

/* Bytes of device scratch ham_decode_step needs (dims->T is ignored). */
size_t ham_decode_workspace_size(const ham_dims *dims);

/*
 * ham_decode_step -- one new token for each of B sequences ([HAM] App. A.1
 * "Generation": the state is carried, routed tokens are appended to the cache).
 * Order within the step: e from S_{t-1}; route; state update; o_rnn; append if
 * routed; attention over the cache including the new entry; mix.  The result
 * equals ham_forward over the same token with HAM_CONTINUE.
 *
 *   q, k, v (+ optional *_attn)  [B,H,dk|dv] io dtype ([B,kv_heads,dk_kv|dv_kv]
 *                                for the attention-path inputs).
 *   beta, g, gate_rnn, gate_kv   [B,H] fp32 ([B,kv_heads] for gate_kv; gates may
 *                                be NULL).
 *   doc_start                    [B] int32 or NULL: absolute start position of
 *                                the new token's document (same-document
 *                                masking, as in ham_forward).
 *   tau                          [H] fp32 ([B,H] with HAM_TAU_PER_TOKEN).
 *   S                            [B,H,dk,dv] fp32, in/out.
 *   Kc, Vc, pos, count           cache of the KV heads, in/out (count <= cap on
 *                                entry).
 *   t_abs                        [B] int32 absolute position of the new token.
 *   o (required), o_rnn, o_kv    [B,H,dv], [B,H,dv], [B,kv_heads,dv_kv] io dtype.
 *   e, routed                    [B,H] or NULL (with HAM_EXTERNAL_SCORES, e is
 *                                the required input score of the new token).
 *   status                       int32 scalar or NULL: set to 1 (never cleared)
 *                                when a routed token found its cache full; the
 *                                append is then skipped.
 *   block_score                  [B,H] fp32, in/out, required when
 *                                dims->route_block > 1 (else ignored, may be
 *                                NULL): the running score sum of each sequence's
 *                                open block.  Block-contiguous routing in decode:
 *                                every token of the open block is written to the
 *                                cache row count + (t_abs mod route_block), past
 *                                count, so it stays invisible; at the block's last
 *                                token the block is decided and, if routed, count
 *                                grows by route_block before that token attends.
 *                                routed is then 1 only at the last token of a
 *                                routed block.  A row that would land at or past
 *                                cap is dropped and status is set.
 */
int ham_decode_step(const ham_dims *dims,
                    const void *q, const void *k, const void *v,
                    const void *q_attn, const void *k_attn, const void *v_attn,
                    const float *beta, const float *g, const float *tau,
                    const float *gate_rnn, const float *gate_kv,
                    const int32_t *doc_start, float *block_score,
                    float *S, void *Kc, void *Vc, int32_t *pos, int32_t *count,
                    const int32_t *t_abs,
                    void *o, void *o_rnn, void *o_kv,
                    float *e, uint8_t *routed, int32_t *status,
                    void *ws, size_t ws_bytes, void *stream);

/*
 * ham_decode_step_noalloc -- ham_decode_step for callers that cannot allocate
 * device memory: code under HIP graph capture, tight serving loops, harnesses
 * that forbid hipMalloc.  Same arguments, semantics, errors and kernels as
 * ham_decode_step, without (ws, ws_bytes): the scratch is a fixed array of
 * HAM_NOALLOC_SCRATCH_BYTES in device memory, one per GPU, which the library
 * holds from the first call on that GPU until the process ends.  Nothing is
 * allocated or freed by the call.
 *   - A step whose ham_decode_workspace_size() exceeds HAM_NOALLOC_SCRATCH_BYTES
 *     is rejected with HAM_EWORKSPACE before anything is enqueued (the split-K
 *     partials need B * kv_heads * ceil(cap / 1024) * (dv_kv + 2) * 4 bytes,
 *     about 9 MiB for batch 32, 16 heads of 128 and a 33K-entry cache).
 *   - Every call on one GPU uses that GPU's one array: calls that overlap on the
 *     same GPU (different streams or threads) race and give wrong results.
 *     Calls on one stream are ordered and safe.
 */
#define HAM_NOALLOC_SCRATCH_BYTES 33554432   /* 32 MiB per GPU */
size_t ham_decode_noalloc_scratch_bytes(void);
int ham_decode_step_noalloc(const ham_dims *dims,
                            const void *q, const void *k, const void *v,
                            const void *q_attn, const void *k_attn, const void *v_attn,
                            const float *beta, const float *g, const float *tau,
                            const float *gate_rnn, const float *gate_kv,
                            const int32_t *doc_start, float *block_score,
                            float *S, void *Kc, void *Vc, int32_t *pos, int32_t *count,
                            const int32_t *t_abs,
                            void *o, void *o_rnn, void *o_kv,
                            float *e, uint8_t *routed, int32_t *status, void *stream);

/* Bytes of device scratch ham_route_stats needs. */
size_t ham_route_stats_workspace_size(const ham_dims *dims);

/*
 * ham_route_stats -- routing only: the RNN over T tokens (no readout, no
 * attention), scores, threshold and counts.  KV usage ([HAM] §5, per layer):
 * rho = sum(count) / (B*T*H).
 *
 *   q, k, v, beta, g, tau, S0    as in ham_forward (q is unused; may be NULL).
 *   e, routed                    optional outputs as in ham_forward.
 *   count                        [B,H] int32, required: tokens routed per head.
 *   n_near                       [H] int64 or NULL: tokens with |e - tau_h| <
 *                                near_band (near-threshold tokens).
 *   rho_host                     HOST double* or NULL; if set, the call waits for
 *                                the stream and stores rho there.
 * HAM_EXTERNAL_SCORES is not accepted (HAM_EUNSUPPORTED): with a learned router
 * the scores do not come from the RNN; ham_select_tau sets a threshold on them.
 */
int ham_route_stats(const ham_dims *dims,
                    const void *q, const void *k, const void *v,
                    const float *beta, const float *g, const float *tau,
                    const float *S0,
                    float *e, uint8_t *routed, int32_t *count,
                    int64_t *n_near, float near_band, double *rho_host,
                    void *ws, size_t ws_bytes, void *stream);

/*
 * ham_select_tau -- per-head threshold for a target KV fraction rho ([HAM] §5:
 * rho_KV, the share of a layer's tokens kept in the KV cache; App. A.1 "Forward
 * Pass": a token is stored when its score exceeds the threshold; one threshold
 * per head here).  For head h, with the N = B*T scores e[:, :, h] and k = rho*N
 * rounded to the nearest integer (ties to even):
 *   tau[h] = +inf when k = 0, -inf when k = N, and otherwise the float nearest to
 *   the midpoint (formed in double) of the (N-k)-th and (N-k+1)-th smallest
 *   scores, NaN sorting above every number.  Exactly k scores then exceed tau[h]
 *   when those two differ; NaN scores never route.
 *
 *   dims   B, T, H (other fields are not read; B*T <= 2^31 - 1).
 *   e      [B,T,H] fp32 device scores (fit-error or learned-router units).
 *   rho    in [0, 1].
 *   tau    [H] fp32 device output.
 * No workspace; one workgroup per head (exact radix select, deterministic).
 * Errors: HAM_EINVAL (NULL pointer, B/T/H <= 0, B*T too large, rho outside
 * [0, 1] or NaN, misaligned pointer), HAM_EHIP.
 */
int ham_select_tau(const ham_dims *dims, const float *e, double rho, float *tau, void *stream);

/* Bytes of device scratch ham_attention_backward needs. */
size_t ham_attention_backward_workspace_size(const ham_dims *dims);

/*
 * ham_attention_backward -- gradients of the KV-memory readout for training ([HAM]
 * §2 KV-memory equation; App. A.1 "FlexAttention and Block Masks" for the visible
 * set): given dO = dL/do_kv, the gradients of softmax attention over the cache,
 *   D_t = dO_t . o_kv_t,  dq_t = scale sum_c p_tc (dO_t . v_c - D_t) k_c,
 *   dk_c = scale sum_t p_tc (dO_t . v_c - D_t) q_t,  dv_c = sum_t p_tc dO_t.
 * The routing threshold passes no gradient.  The visible set is read from the
 * cache: query t (position t0 + t) sees the entries at positions <= t0 + t (and,
 * with doc_start, >= its document's start), so the cache may hold entries of
 * earlier calls.  Acts on the KV heads (kv_heads, dk_kv, dv_kv: 64 or 128 each).
 *
 *   q_attn             [B,T,kv_heads,dk_kv] io dtype: the queries of the forward.
 *   Kc, Vc, pos, count the cache as the forward left it.
 *   doc_start          [B,T] int32 or NULL, as in ham_forward.
 *   dO                 [B,T,kv_heads,dv_kv] fp32: dL/do_kv.
 *   dq                 [B,T,kv_heads,dk_kv] fp32 out.
 *   dKc, dVc           [B,kv_heads,cap,dk_kv|dv_kv] fp32 out, entries < count
 *                      (the caller scatters them to token positions through pos).
 * Errors: HAM_EINVAL, HAM_EUNSUPPORTED (rope_base > 0, route_block > 1, or KV
 * sizes other than 64/128), HAM_EWORKSPACE, HAM_EHIP.
 */
int ham_attention_backward(const ham_dims *dims, const void *q_attn, const void *Kc, const void *Vc,
                           const int32_t *pos, const int32_t *count, const int32_t *doc_start,
                           const float *dO, float *dq, float *dKc, float *dVc,
                           void *ws, size_t ws_bytes, void *stream);

/* Bytes of device scratch ham_rnn_backward needs (0 on bad or unsupported dims). */
size_t ham_rnn_backward_workspace_size(const ham_dims *dims);

/*
 * ham_rnn_backward -- gradients of the gated delta-rule RNN for training ([HAM]
 * §2 DeltaNet update and linear-attention readout, App. A.1 gated DeltaNet; the
 * pages train the layer end to end).  Per head, with alpha_t = exp(g_t),
 *   p_t = S_{t-1}^T k_t, r_t = v_t - alpha_t p_t, S_t = alpha_t S_{t-1} + beta_t k_t r_t^T,
 *   o_rnn_t = S_t^T q_t,
 * given dO = dL/do_rnn and dS_T = dL/dS_T, the gradients with respect to q, k, v,
 * beta, g and the entering state (reverse mode of that recurrence, fp32).  It runs
 * chunked ([HAM] App. A.1: the chunked kernel also serves the backward pass): reverse
 * mode of the 64-token chunk form of the forward state pass, a forward and a reverse
 * chain over the chunks and chunk-parallel gradient terms; with HAM_FORCE_RECURRENT
 * in dims->flags, token by token instead.  The routing decision passes no gradient;
 * the gradient of the mix (norms, gates) and of the attention
 * (ham_attention_backward) are separate.
 *
 *   dims               B, T, H, dk, dv (64 or 128 each), io_dtype, flags
 *                      (HAM_FORCE_RECURRENT or 0); other fields are not read.
 *   q, k, v            [B,T,H,dk|dv] io dtype: the forward's RNN inputs.
 *   beta, g            [B,T,H] fp32.
 *   S0                 [B,H,dk,dv] fp32 entering state of the forward, or NULL (0).
 *   dO                 [B,T,H,dv] fp32, required.
 *   dS_T               [B,H,dk,dv] fp32 or NULL (0).
 *   dq, dk, dv         [B,T,H,dk|dv] fp32 out;  dbeta, dg [B,T,H] fp32 out;
 *   dS0                [B,H,dk,dv] fp32 out: dL/dS0.
 *   ws, ws_bytes       scratch of ham_rnn_backward_workspace_size(dims) bytes
 *                      (the same flags): chunked, the entering state and its
 *                      gradient at every chunk and per-chunk matrices (about
 *                      2 x T/64 states and (4 d_v + 192) T floats per head);
 *                      token by token, the state at every chunk start and one
 *                      chunk's states per 16 state columns.
 * Errors: HAM_EINVAL, HAM_EUNSUPPORTED (dk or dv not 64/128), HAM_EWORKSPACE,
 * HAM_EHIP.
 */
int ham_rnn_backward(const ham_dims *dims, const void *q, const void *k, const void *v,
                     const float *beta, const float *g, const float *S0,
                     const float *dO, const float *dS_T,
                     float *dq, float *dk, float *dv, float *dbeta, float *dg, float *dS0,
                     void *ws, size_t ws_bytes, void *stream);

/*
 * Instrumentation (not part of the method): HIP-event timing of the kernel
 * stages of the next calls.  ham_profile_start(max_calls) arms recording on the
 * current device for up to max_calls subsequent ham_forward / ham_decode_step /
 * ham_route_stats calls (any thread; events are recorded on each call's own
 * stream around each kernel launch).  ham_profile_stop waits for the recorded
 * events and writes stage_ms[call * HAM_PROFILE_STAGES + stage] (milliseconds,
 * 0 for unused stages) for at most max_values values, the number of recorded
 * calls to *n_calls and each call's entry point to kinds[call] (0 forward,
 * 1 decode, 2 route_stats; kinds may be NULL).  Stages: forward {rnn_prep,
 * rnn_state, route, compact, attention}; decode {rnn, route, append, attention,
 * combine}; route_stats {rnn_prep, rnn_state, route, stats}.  rnn_prep is the
 * chunk-parallel part of the chunked recurrence (0 on the token-serial path).
 * Returns HAM_OK, HAM_EINVAL or HAM_EHIP.
 */
#define HAM_PROFILE_STAGES 5
int ham_profile_start(int max_calls);
int ham_profile_stop(float *stage_ms, int max_values, int *n_calls, int *kinds);

#ifdef __cplusplus
}
#endif
#endif /* HAM_H */
