/*
 * moe_verify.h - C ABI of the MI355X (gfx950) MoE verify-step library.
 *
 * The verify step is the hot path of FastMTP speculative decoding on a
 * mixture-of-experts decoder, as described on "Jina AI Releases jina-ocr-v1,
 * a 3.4B MoE Document Parser With Built-In Speculative Decoding"
 * (ainewsfeed.tech):
 *   - architecture paragraph: the decoder stacks MoE layers with 64 routed
 *     experts, two shared experts and top-6 routing;
 *   - FastMTP paragraph: the decoder verifies K drafts greedily, accepts the
 *     longest prefix matching its own choices and commits one more token
 *     itself (a bonus token when all K matched), so the committed text equals
 *     plain greedy decoding.
 * The modelscope.ai page "Jina-OCR-v1: Efficient Document Parsing with
 * Speculative Decoding and Dense Verifiable Rewards" (Abstract) gives K = 3.
 * Attention is not part of this library: each token row is independent.
 *
 * Conventions for every entry point
 *   - Every tensor pointer is DEVICE memory owned by the caller, which keeps
 *     it alive until the work enqueued on `stream` has completed.  The library
 *     allocates, frees and synchronises nothing; all work is enqueued on
 *     `stream` (a hipStream_t; NULL means the default stream).
 *   - Matrices are row-major, [out, in] like a torch Linear weight.
 *     Elements of weights and hidden states are in the config's dtype:
 *     fp32, or bf16 (raw 16-bit patterns).  Logits, gates and every
 *     accumulator are fp32; bf16 rounding (to nearest even) happens only
 *     where a value is stored in the model dtype: the hidden state between
 *     layers, the normalised layer input x, the SwiGLU product, and the
 *     final normalised x_f.
 *   - Arguments are validated on the host before anything is enqueued.  On
 *     error the call returns a negative MV_ERR_* code, enqueues nothing and
 *     sets a thread-local message readable with mv_last_error().
 *   - Zero tokens (T = 0 or B = 0) is valid and does nothing.
 *   - Calls are reentrant; two calls that share a workspace must not overlap
 *     on the GPU.
 */
#ifndef MOE_VERIFY_H
#define MOE_VERIFY_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum { MV_F32 = 0, MV_BF16 = 1 };

enum {
  MV_OK = 0,
  MV_ERR_NULL = -1,        /* a required pointer is NULL                     */
  MV_ERR_SHAPE = -2,       /* negative or too large T/B/K, bad layer index   */
  MV_ERR_UNSUPPORTED = -3, /* config outside what the kernels implement      */
  MV_ERR_WORKSPACE = -4,   /* workspace smaller than mv_workspace_bytes()    */
  MV_ERR_HIP = -5          /* a HIP launch reported an error                 */
};

/* Model shape.  Supported: d_model and d_ff multiples of 64, d_model <= 4096,
 * d_ff <= 8192, 1 <= top_k <= min(8, n_routed), 1 <= n_routed <= 64,
 * 0 <= n_shared <= 4, n_layers >= 1, vocab >= 1, rms_eps > 0,
 * dtype MV_F32 or MV_BF16. */
typedef struct {
  int32_t d_model;  /* d: hidden width                                     */
  int32_t d_ff;     /* F: FFN width of one expert                          */
  int32_t n_routed; /* E: routed experts per layer                         */
  int32_t n_shared; /* S: always-on shared experts per layer (gate 1)      */
  int32_t top_k;    /* k: routed experts chosen per token                  */
  int32_t n_layers; /* L: MoE layers                                       */
  int32_t vocab;    /* V: LM-head rows                                     */
  float rms_eps;    /* RMSNorm epsilon                                     */
  int32_t dtype;    /* MV_F32 or MV_BF16                                   */
} mv_config;

/* Weights, all in the config dtype except router_b (fp32).  Per layer l:
 *   ffn_norm   [L, d]         RMSNorm scale before the MoE
 *   router_w   [L, E, d]      router logits l = x W_r^T (+ b)
 *   router_b   [L, E] fp32    optional additive router bias (NULL: none)
 *   w_gate_up  [L, E, 2F, d]  rows [0, F) gate, [F, 2F) up; one expert's
 *                             block is contiguous
 *   w_down     [L, E, d, F]
 *   ws_gate_up [L, S, 2F, d]  shared experts, same layout (NULL if S = 0)
 *   ws_down    [L, S, d, F]
 *   final_norm [d]            RMSNorm scale before the LM head
 *   lm_head    [V, d]
 */
typedef struct {
  const void *ffn_norm;
  const void *router_w;
  const float *router_b;
  const void *w_gate_up;
  const void *w_down;
  const void *ws_gate_up;
  const void *ws_down;
  const void *final_norm;
  const void *lm_head;
} mv_weights;

/* Bytes of device workspace a call with up to `max_tokens` token rows needs
 * (256-byte aligned pointer expected).  Host-only, pure; returns 0 for an
 * invalid config or max_tokens outside [0, 65535]. */
size_t mv_workspace_bytes(const mv_config *cfg, int32_t max_tokens);

/* One MoE layer for T token rows (architecture paragraph of the ainewsfeed
 * page: 64 routed experts, top-6 routing, two shared experts):
 *   x   = bf16(RMSNorm(h_in) * ffn_norm[layer])
 *   l   = x router_w[layer]^T (+ router_b[layer])            fp32
 *   ids = the top_k experts by (logit desc, expert id asc), in that order
 *   w   = softmax over the top_k selected logits             fp32
 *   y   = sum_s w_s FFN_{ids_s}(x) + sum_shared FFN_shared(x) (fp32, that order)
 *   FFN_e(x) = (bf16(SiLU(x Wg_e^T) * (x Wu_e^T))) Wd_e^T
 *   h_out = bf16(h_in + y)
 * h_in, h_out: [T, d] in the config dtype; h_out may alias h_in.
 * topk_ids [T, k] int32, topk_w [T, k] fp32, y_moe [T, d] fp32: optional
 * outputs (NULL to skip).  ws: >= mv_workspace_bytes(cfg, T) bytes. */
int moe_layer_forward(const mv_config *cfg, const mv_weights *w, int32_t layer,
                      int32_t T, const void *h_in, void *h_out,
                      int32_t *topk_ids, float *topk_w, float *y_moe,
                      void *ws, size_t ws_bytes, void *stream);

/* One verify step for B sequences with K drafts each (FastMTP paragraph of
 * the ainewsfeed page).  T = B*(K+1) rows: row b*(K+1) is the hidden state
 * of sequence b's last committed token, rows b*(K+1)+1..K those of its
 * drafts.  All n_layers layers run as in moe_layer_forward, then
 *   x_f = bf16(RMSNorm(h) * final_norm), z = x_f lm_head^T (fp32, never
 *   stored), argmax[t] = lowest id among the maximal z[t].
 * Accept (per sequence): n = first j in [0, K) with drafts[b,j] !=
 * argmax[b,j], else K; committed[b, 0..n] = argmax[b, 0..n], the rest -1;
 * n_accepted[b] = n; n_committed[b] = n + 1 (bonus token when n = K).
 * Draft ids outside [0, V) are not an error; they never match.
 *   h_in      [T, d]      config dtype
 *   drafts    [B, K]      int32 (may be NULL when K = 0)
 *   h_out     [T, d]      hidden state after the last layer, before the final
 *                         norm (NULL to skip); may alias h_in
 *   argmax    [T]         int32
 *   n_accepted, n_committed [B] int32;  committed [B, K+1] int32
 *   dbg_topk_ids [L, T, k] int32 routing of every layer (NULL to skip)
 * Limits: 0 <= K <= 15, T <= 65535. */
int moe_verify_step(const mv_config *cfg, const mv_weights *w, int32_t B,
                    int32_t K, const void *h_in, const int32_t *drafts,
                    void *h_out, int32_t *argmax, int32_t *n_accepted,
                    int32_t *committed, int32_t *n_committed,
                    int32_t *dbg_topk_ids, void *ws, size_t ws_bytes,
                    void *stream);

/* moe_verify_step as one launch (throughput paragraph of the ainewsfeed page:
 * removing per-step launch overhead with graph replay lifted plain greedy
 * decoding from 42.7 to 158.3 tokens/s on an L4).  For batches of at most 8
 * rows (B*(K+1) <= 8) and at most 16 layers; arguments, results and
 * workspace as in moe_verify_step, and the results are bit-identical to it.
 * A small setup kernel writes the step's arguments into the workspace and
 * clears its counters; one launch then runs every layer's routing and
 * experts, the final norm and the LM head with the accept rule, its blocks
 * in step order, so that the next layer's shared experts and the LM head can
 * stream their weights while the previous stage finishes.  Errors: larger
 * batches or more layers MV_ERR_UNSUPPORTED.  A wait that gives up sets the
 * status word (mv_step_status), as in moe_verify_step. */
int moe_verify_step_one_launch(const mv_config *cfg, const mv_weights *w, int32_t B,
                               int32_t K, const void *h_in, const int32_t *drafts,
                               void *h_out, int32_t *argmax, int32_t *n_accepted,
                               int32_t *committed, int32_t *n_committed,
                               int32_t *dbg_topk_ids, void *ws, size_t ws_bytes,
                               void *stream);

/* moe_verify_step for callers that cannot allocate device memory: code under
 * HIP graph capture, tight serving loops, harnesses that forbid allocation.
 * Arguments and results as in moe_verify_step, without ws and ws_bytes: the
 * workspace is a static 16 MiB array of the library, one per GPU, looked up
 * (not allocated) on the first call on that GPU and held until the process
 * ends.  The call allocates nothing.  Steps whose workspace
 * (mv_workspace_bytes(cfg, B*(K+1))) exceeds 16 MiB are rejected with
 * MV_ERR_WORKSPACE: about 250 rows at d_model 1280, d_ff 896, 64 + 2
 * experts, top-6 (B = 32, K = 3 takes 8.1 MiB).  Every call on one GPU uses
 * the same array and leaves its contents behind; the kernels clear what must
 * start at zero, so consecutive calls are independent, but two calls that
 * overlap on one GPU (other streams, other threads) race.  mv_step_status
 * with ws = NULL reads this array's status word. */
int moe_verify_step_noalloc(const mv_config *cfg, const mv_weights *w, int32_t B,
                            int32_t K, const void *h_in, const int32_t *drafts,
                            void *h_out, int32_t *argmax, int32_t *n_accepted,
                            int32_t *committed, int32_t *n_committed,
                            int32_t *dbg_topk_ids, void *stream);

/* The accept rule alone (FastMTP paragraph of the ainewsfeed page), on
 * argmax [B, K+1] and drafts [B, K]; outputs as in moe_verify_step.
 * Limits: 0 <= K <= 15.  No workspace. */
int spec_accept(int32_t B, int32_t K, const int32_t *argmax,
                const int32_t *drafts, int32_t *n_accepted,
                int32_t *committed, int32_t *n_committed, void *stream);

/* FastMTP draft block (FastMTP paragraph of the ainewsfeed page: one dense
 * block whose parameters are shared by every draft position, drafting
 * through the decoder's own LM head).  The block's inner layers are not on
 * the pages; this library uses the plainest reading.  Weights in the config
 * dtype, [out, in] row-major:
 *   embed     [V, d]      token embeddings
 *   norm_h    [d]         RMSNorm scale of the incoming hidden state
 *   norm_e    [d]         RMSNorm scale of the token's embedding
 *   w_proj    [d, 2d]     projection of [norm(h) ; norm(e)]
 *   norm_ffn  [d]         RMSNorm scale before the dense FFN
 *   w_gate_up [2Fm, d]    rows [0, Fm) gate, [Fm, 2Fm) up
 *   w_down    [d, Fm]
 *   norm_out  [d]         RMSNorm scale before the LM head
 *   d_ff      Fm: a positive multiple of 64 */
typedef struct {
  const void *embed;
  const void *norm_h;
  const void *norm_e;
  const void *w_proj;
  const void *norm_ffn;
  const void *w_gate_up;
  const void *w_down;
  const void *norm_out;
  int32_t d_ff;
} mtp_weights;

/* Bytes of device workspace mtp_draft needs for up to max_rows sequences
 * (256-byte aligned pointer expected).  Host-only, pure; 0 for an invalid
 * config, an unsupported width or max_rows outside [0, 65535]. */
size_t mtp_workspace_bytes(const mv_config *cfg, int32_t d_ff_mtp, int32_t max_rows);

/* K draft tokens for each of B sequences.  Per sequence, from its hidden
 * state h (the decoder's last hidden state, before the final norm, as
 * moe_verify_step's h_out returns it) and the token t that follows it:
 *   u  = [ R(RMSNorm(h) * norm_h) ; R(RMSNorm(embed[t]) * norm_e) ]
 *   h1 = R(u w_proj^T)
 *   h2 = R(h1 + (R(SiLU(x Wg^T) * (x Wu^T))) w_down^T),  x = R(RMSNorm(h1) * norm_ffn)
 *   draft = lowest id among the maximal z,  z = R(RMSNorm(h2) * norm_out) lm_head^T
 * R() rounds to the config dtype; every sum is fp32.  The next draft applies
 * the same block to (h2, draft).
 *   w         decoder weights; only lm_head is read
 *   h_in      [B, d]  config dtype
 *   tokens    [B]     int32; an id outside [0, V) is clamped into it
 *   drafts    [B, K]  int32
 *   h_out     [B, d]  the block's last h2 (NULL to skip); may alias h_in
 * Limits: 0 <= K <= 15, B <= 65535; the projection and the dense FFN stage
 * 16 rows of width 2d and d_ff in LDS: d_model <= 2112 and d_ff <= 4800 in
 * bf16, d_model <= 1024 and d_ff <= 2368 in fp32 (MV_ERR_UNSUPPORTED beyond).
 * K = 0 or B = 0 does nothing. */
int mtp_draft(const mv_config *cfg, const mv_weights *w, const mtp_weights *m, int32_t B,
              int32_t K, const void *h_in, const int32_t *tokens, int32_t *drafts,
              void *h_out, void *ws, size_t ws_bytes, void *stream);

/* Draft length for the next speculative step (FastMTP paragraph of the
 * ainewsfeed page: the best K depends on acceptance and on what a step
 * costs).  With K drafts, each accepted independently with probability q,
 * the accept rule commits E(K) = 1 + q + ... + q^K tokens per sequence on
 * average; the chosen K in [0, k_max] maximises E(K) / cost[K], the smallest
 * K on ties.  cost[K] (host memory, k_max + 1 values, each > 0) is the cost
 * of one step with K drafts in any unit: measured time, or mv_step_bytes.
 *   k_best  the chosen K;  rate  E(k_best) / cost[k_best] (NULL to skip)
 * Host-only, pure.  Errors: MV_ERR_NULL, MV_ERR_SHAPE (k_max outside
 * [0, 15], q outside [0, 1], a cost not > 0). */
int mv_choose_k(int32_t k_max, float q, const float *cost, int32_t *k_best, float *rate);

/* Expected HBM bytes of one speculative step for B sequences with K drafts:
 * K positions of the draft block (its matrices, the LM head, four norm
 * vectors, and per sequence the embedding row and hidden rows in and out;
 * d_ff_mtp = 0 for no draft block), then moe_verify_step over T = B (K+1)
 * rows (all routed experts the rows choose, with uniform routing an expert
 * is chosen by some row with probability 1 - (1 - top_k / n_routed)^T; the
 * shared experts, router and norm vectors, the LM head, the rows in and
 * out).  Host-only, pure; a negative value on invalid arguments. */
double mv_step_bytes(const mv_config *cfg, int32_t B, int32_t K, int32_t d_ff_mtp);

/* Status of the last moe_verify_step or moe_layer_forward call made on the
 * workspace ws.  Calls of up to 8 token rows run each layer's routing, gate/up
 * and down in one launch, whose blocks wait on counters that blocks of lower
 * index raise; those blocks are dispatched first, so the waits end.  Each
 * wait is nonetheless bounded (mv_set_spin_limit): one that gives up lets
 * its block go on with whatever data it finds, and records 1 in a status
 * word at offset 0 of the workspace, which the first launch of every call
 * clears.  This call enqueues, on `stream`, a copy of that word into
 * status[0] (device memory, int32): 0 means every wait of the call ended as
 * it should; 1 means the call's results must not be used.  ws = NULL reads
 * the current GPU's static workspace of moe_verify_step_noalloc.  Errors:
 * MV_ERR_NULL (status NULL), MV_ERR_WORKSPACE (ws not 256-byte aligned). */
int mv_step_status(const void *ws, int32_t *status, void *stream);

/* Test hook for the bounded waits above: the number of polls (each about a
 * microsecond) a wait makes before it gives up, for calls enqueued after
 * this one, process-wide.  polls < 0 restores the default (2^18); polls = 0
 * makes every wait that finds its counter short give up at once.  Returns
 * the previous limit.  Host-only; every kernel still runs to its end
 * whatever the limit. */
int32_t mv_set_spin_limit(int32_t polls);

/* Message of the last error on the calling thread ("" if none). */
const char *mv_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* MOE_VERIFY_H */
