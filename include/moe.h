/*
 * moe.h -- C ABI of the MI355X (gfx950) forward pass of one
 * Mixture-of-Experts FFN layer.
 *
 * The layer ("DeepSpeed MoE and Model Compression", section "DeepSpeed-MoE",
 * its equation and its pipeline block):
 *   p(x)  = softmax(W_r x (+ b_r))                      router
 *   ids   = the k largest p, descending, ties -> lower expert index
 *   gates = p of the chosen experts (k >= 2: renormalised over the k)
 *   dispatch into an expert-major capacity buffer [E, C, d], in token order,
 *   C = min(T, ceil(k*T*cf/E)); assignments past C are dropped
 *   ("DeepSpeed-MoE vs Switch Transformer", section "expert capacity overflow")
 *   expert FFN  y_e = W2_e GELU(W1_e x)   (survey notes sec. 1.1.2.1)
 *   y = [x] + [dense MLP(x)] + sum over kept j of gates_j y_{e_j}
 *   (PR-MoE, "DeepSpeed-MoE ... notes" sec. 3.1)
 *   aux = alpha * E * sum_i f_i Q_i   (survey notes sec. 1.1.4.1)
 *
 * Conventions for every entry point
 *   - Every tensor pointer is a DEVICE pointer owned by the caller, row-major,
 *     16-byte aligned.  Weights are [out, in]: W_r [E, d], W1 [E, d_ff, d],
 *     W2 [E, d, d_ff], Wm1 [d_ff_dense, d], Wm2 [d, d_ff_dense].
 *   - "act" = the configuration's activation type (MOE_F32 or MOE_BF16); it is
 *     the type of x, W_r, plain expert weights, the dense MLP weights, x_disp,
 *     y_disp and y.  ids/slots/load/kept are int32, gates/logits/aux float32,
 *     drop masks uint8, int8 scales IEEE fp16.
 *   - `stream` is a hipStream_t (NULL = the default stream).  Calls only
 *     enqueue work: no host synchronisation, no allocation, no host<->device
 *     copies.  Results are valid once the stream has been synchronised.
 *   - Scratch memory comes from the caller's workspace `ws` of at least
 *     moe_workspace_bytes(cfg, entry) bytes (256-byte aligned).
 *   - Arguments are validated before anything is enqueued; on error nothing
 *     is launched and no output is written.  Return 0 (MOE_OK) or a negative
 *     MOE_ERR_* code; moe_status_string() names it.
 *   - Results are deterministic: the same inputs give bit-identical outputs.
 *   - Apart from the optional timing records (moe_profile_*) and the side
 *     stream below, the library keeps no state between calls; calls on
 *     different streams with disjoint buffers may run concurrently.
 *   - moe_layer_forward with pr_moe and overlap_dense runs the dense MLP on a
 *     library-owned side stream (non-blocking, default priority; one per
 *     device, created with its two events on the first such call and kept
 *     until the process ends), forked from and joined back into `stream`
 *     with events, so the call stays asynchronous and ordered on `stream` as
 *     a whole.
 */
#ifndef MOE_MI355X_H
#define MOE_MI355X_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* status codes */
#define MOE_OK 0
#define MOE_ERR_INVALID_ARG (-1) /* null required pointer, bad size, misaligned */
#define MOE_ERR_UNSUPPORTED (-2) /* a valid configuration this build does not run */
#define MOE_ERR_WORKSPACE (-3)   /* workspace missing or smaller than required */
#define MOE_ERR_HIP (-4)         /* the HIP runtime reported an error at launch */
#define MOE_ERR_SCRATCH (-5)     /* moe_layer_forward_noalloc: the configuration needs
                                    more than MOE_NOALLOC_SCRATCH_BYTES of scratch */

/* Size of the library's own per-device scratch array that
 * moe_layer_forward_noalloc uses instead of a caller workspace (32 MiB). */
#define MOE_NOALLOC_SCRATCH_BYTES (32u << 20)

/* activation types */
#define MOE_F32 0
#define MOE_BF16 1

/* expert weight formats */
#define MOE_W_PLAIN 0     /* act type */
#define MOE_W_INT8_G128 1 /* symmetric int8 codes q, fp16 scale s per 128
                             consecutive input-dim elements of an output row;
                             weight = s * q (survey notes sec. 1.2.2) */
#define MOE_W_BF16_PACKED 2 /* bf16 weights of an [E, N, K] expert matrix
                               in blocks of 128 output rows x 64 inputs:
                               element (e, n, k) sits at e*N*K +
                               (n/128)*128*K + (k/64)*8192 + (n%128)*64 +
                               k%64, so each 64-wide K step of a 128-row
                               block is 16 KB of contiguous memory (the
                               weight stream of the expert GEMMs reads whole
                               blocks).  bf16 activations, d and d_ff
                               multiples of 128; forward entry points only.
                               moe_pack_expert_weights writes it. */

/* capacity overflow policy */
#define MOE_DROP_TOKEN_ORDER 0   /* first come, first served in token order */
#define MOE_DROP_GATE_PRIORITY 1 /* an expert keeps the C assignments with the
                                    largest gates, ties to the earlier token;
                                    slot = rank in that order ("DeepSpeed-MoE
                                    vs Switch Transformer", capacity example in
                                    which the lower-probability token is the
                                    one dropped) */

/* workspace query selectors */
/* router (moe_config.router), the MoE survey notes' gating variants:
 *  TOPK     p = softmax(W_r x + b), the k largest p (the default above)
 *  TOP_P    p as TOPK; experts in descending p, accumulated until their sum
 *           exceeds top_p, at most k of them (sec. 1.1.4.2); a token's unused
 *           slots have expert id -1 and gate 0 and are no assignment; gates
 *           renormalised over the taken experts when normalize_topk
 *  COSINE   logit_e = <emb_e, W_proj x> / (cos_tau |W_proj x| |emb_e|) (+ b),
 *           0 when a norm is 0 (sec. 1.1.1.2); then as TOPK
 *  NOISY_TOPK  clean = W_r x + b, sigma = softplus(W_noise x), logit =
 *           clean + noise * sigma with the caller's standard-normal draws; the
 *           k largest logits kept, gates = softmax over them (sec. 1.1.1.1)
 * Every router can also report the Importance and Load losses (sec. 1.1.4.1):
 *   w_importance * CoV(sum_t gate_e)^2 and w_load * CoV(sum_t P(x_t, e))^2,
 *   CoV^2 = population variance / mean^2 over the experts (0 for mean 0),
 *   P(x, e) = Phi((clean_e - k-th largest logit among the other experts) /
 *   sigma_e) for NOISY_TOPK (the probability that e keeps a nonzero gate
 *   under a new draw of its noise), else 1 if e was chosen and 0 if not. */
#define MOE_ROUTER_TOPK 0
#define MOE_ROUTER_TOP_P 1
#define MOE_ROUTER_COSINE 2
#define MOE_ROUTER_NOISY_TOPK 3

#define MOE_ENTRY_ROUTE 0
#define MOE_ENTRY_DISPATCH 1
#define MOE_ENTRY_EXPERT_FFN 2
#define MOE_ENTRY_COMBINE 3
#define MOE_ENTRY_LAYER 4
#define MOE_ENTRY_BACKWARD 5

/* Sizes: with MOE_BF16 activations d, d_ff and (PR-MoE) d_ff_dense must be
 * multiples of 64, and with int8 or packed expert weights d and d_ff
 * multiples of 128; other values return MOE_ERR_UNSUPPORTED.  MOE_F32 takes
 * any positive sizes. */
typedef struct moe_config {
  int64_t T;          /* tokens (>= 0) */
  int64_t d;          /* model dim (>= 1; bf16: a multiple of 64) */
  int64_t E;          /* experts, 1..256 */
  int64_t k;          /* experts per token, 1..min(E, 8) */
  int64_t d_ff;       /* expert hidden dim (>= 1; bf16: a multiple of 64) */
  int64_t d_ff_dense; /* PR-MoE dense MLP hidden dim (used when pr_moe;
                         bf16: a multiple of 64) */
  double capacity_factor; /* > 0; C = min(T, ceil(k*T*cf/E)) */
  int64_t capacity;       /* > 0 overrides the formula (still clamped to T) */
  int32_t act_dtype;      /* MOE_F32 | MOE_BF16 */
  int32_t expert_wfmt;    /* MOE_W_PLAIN | MOE_W_INT8_G128 | MOE_W_BF16_PACKED
                             (the last two: bf16 acts only) */
  int32_t normalize_topk; /* k >= 2: 1 = gates renormalised over the k */
  int32_t pr_moe;         /* 1 = add the fixed dense MLP D(x) */
  int32_t add_skip;       /* 1 = add x (the residual a dropped token rides) */
  int32_t drop_policy;    /* MOE_DROP_TOKEN_ORDER | MOE_DROP_GATE_PRIORITY */
  float aux_alpha;        /* alpha of the load-balance loss */
  int32_t overlap_dense;  /* pr_moe, moe_layer_forward: 1 = run the dense MLP on
                             the library's side stream, concurrently with the
                             expert path; 0 = everything in order on `stream` */
  int32_t router;         /* MOE_ROUTER_* (0 = TOPK) */
  float top_p;            /* TOP_P: threshold P > 0 */
  float cos_tau;          /* COSINE: temperature > 0 */
  int32_t cos_dim;        /* COSINE: projection width 1..256 */
  float w_importance;     /* Importance-loss weight (0 = not computed) */
  float w_load;           /* Load-loss weight (0 = not computed) */
  int32_t read_x_rows;    /* moe_layer_forward: 0 (default) = the gather builds
                             the explicit [E, C, d] buffer x_disp that the first
                             expert GEMM reads; 1 = when x_disp is not among the
                             outputs (and with token-order dispatch, bf16
                             activations and expert shapes on the DMA tiles),
                             the first expert GEMM reads the token rows of x
                             through the slot -> token table instead and no
                             gathered copy is made (same results, bit for bit) */
} moe_config;

typedef struct moe_weights {
  const void *w_router;  /* [E, d] act */
  const float *b_router; /* [E] or NULL (a logit bias, included in p) */
  const void *w1;        /* [E, d_ff, d] act or int8 */
  const void *w1_scale;  /* [E, d_ff, d/128] fp16 (int8 only, else NULL) */
  const void *w2;        /* [E, d, d_ff] act or int8 */
  const void *w2_scale;  /* [E, d, d_ff/128] fp16 (int8 only, else NULL) */
  const void *wm1;       /* [d_ff_dense, d] act (pr_moe only) */
  const void *wm2;       /* [d, d_ff_dense] act (pr_moe only) */
  /* router variants (NULL unless the router needs them): */
  const void *w_noise;   /* NOISY_TOPK: [E, d] act */
  const void *w_proj;    /* COSINE: [cos_dim, d] act (w_router unused) */
  const void *expert_emb;/* COSINE: [E, cos_dim] act */
  const float *noise;    /* NOISY_TOPK: [T, E] fp32 standard-normal draws of this
                            call (an input, not a weight) */
} moe_weights;

typedef struct moe_outputs {
  void *y;             /* [T, d] act                           required */
  int32_t *expert_ids; /* [T, k]                                required */
  float *gates;        /* [T, k]                                required */
  int32_t *slots;      /* [T, k] slot in the expert, -1 dropped required */
  int32_t *load;       /* [E] assignments received              required */
  int32_t *kept;       /* [E] min(load, C)                      required */
  float *aux_loss;     /* [1]                                   required */
  uint8_t *drop_mask;  /* [T, k] 1 = dropped                    optional */
  float *logits;       /* [T, E] router logits (+ bias)         optional */
  void *x_disp;        /* [E, C, d] act; NULL = in the workspace (or, with
                          cfg->read_x_rows, not built: see moe_config) */
  void *y_disp;        /* [E, C, d] act; NULL = in the workspace */
  void *dense_out;     /* [T, d] act D(x) (pr_moe); NULL = workspace */
  float *z_loss;       /* [1] router z-loss                     optional */
  /* Activations a training forward keeps for moe_layer_backward (each
   * optional; the rows past an expert's kept count are not written):   */
  void *h_disp;        /* [E, C, d_ff] act GELU(W1 x) of the kept rows; NULL = workspace */
  void *z_disp;        /* [E, C, d_ff] act W1 x, the pre-activation; NULL = not kept */
  void *h_dense;       /* [T, d_ff_dense] act GELU(Wm1 x) (pr_moe); NULL = workspace */
  void *z_dense;       /* [T, d_ff_dense] act Wm1 x (pr_moe); NULL = not kept */
  float *importance_loss; /* [1] (needs w_importance != 0)     optional */
  float *load_loss;       /* [1] (needs w_load != 0)           optional */
} moe_outputs;

typedef struct moe_grads {
  void *dx;          /* [T, d] act                                  required */
  void *dw_router;   /* [E, d] act                                  required */
  float *db_router;  /* [E] fp32                                    optional */
  void *dw1;         /* [E, d_ff, d] act                            required */
  void *dw2;         /* [E, d, d_ff] act                            required */
  void *dwm1;        /* [d_ff_dense, d] act                 pr_moe: required */
  void *dwm2;        /* [d, d_ff_dense] act                 pr_moe: required */
} moe_grads;

/* Capacity C of the configuration, or a negative MOE_ERR_* code. */
int64_t moe_capacity(const moe_config *cfg);

/* Workspace bytes an entry point needs (MOE_ENTRY_*); 0 for an invalid
 * configuration. */
size_t moe_workspace_bytes(const moe_config *cfg, int entry);

/* Router, softmax, top-k gate and load-balance loss ("DeepSpeed-MoE vs Switch
 * Transformer", section "router computation"; survey notes sec. 1.1.1.1 and
 * 1.1.4.1).  x [T, d], w_router [E, d] act; b_router [E] or NULL.
 * Out: expert_ids [T, k], gates [T, k], logits [T, E] (NULL = not written),
 * aux_loss [1], z_loss [1] (NULL = not computed): the router z-loss
 * ("DeepSpeed-MoE vs Switch Transformer", section "Router Z-loss"), the mean
 * over tokens of the squared log-sum-exp of the token's logits (+ bias).
 * Logits accumulate in fp32; the log-sum-exp is fp32 per token, the mean is
 * summed in fp64 in a fixed order.  The softmax TopK router only
 * (cfg->router == MOE_ROUTER_TOPK, else MOE_ERR_UNSUPPORTED; moe_route_ex
 * runs every router). */
int moe_route(const moe_config *cfg, const void *x, const void *w_router,
              const float *b_router, int32_t *expert_ids, float *gates,
              float *logits, float *aux_loss, float *z_loss, void *ws,
              size_t ws_bytes, void *stream);

/* Any router of moe_config.router (see MOE_ROUTER_*): reads x and the
 * router's members of w (w_router, b_router; w_noise and noise; w_proj and
 * expert_emb); writes out->expert_ids, gates, aux_loss and, when given,
 * logits (the logits the softmax saw: + bias, + noise), z_loss,
 * importance_loss and load_loss (each loss needs its weight != 0).  The
 * other members of out are not touched.  Workspace:
 * moe_workspace_bytes(cfg, MOE_ENTRY_ROUTE). */
int moe_route_ex(const moe_config *cfg, const void *x, const moe_weights *w,
                 moe_outputs *out, void *ws, size_t ws_bytes, void *stream);

/* Capacity-limited dispatch and the layout transform into the expert-major
 * buffer ("DeepSpeed MoE and Model Compression", pack_by_expert;
 * "DeepSpeed-MoE ... notes" sec. 4.4 cumsum mapping table and layout
 * transformation).  x [T, d], expert_ids [T, k]; gates [T, k] fp32 (used by
 * MOE_DROP_GATE_PRIORITY, where it is required and must be finite; may be
 * NULL for MOE_DROP_TOKEN_ORDER).
 * An expert id outside 0..E-1 (an unused TopP slot) is no assignment:
 * slot -1, drop_mask 0, not counted in load.
 * Out: slots [T, k] (-1 = dropped), drop_mask [T, k] (NULL ok), load [E],
 * kept [E], x_disp [E, C, d]: row (e, s) = x[t] for the assignment with slot
 * s in expert e; rows s >= kept[e] are not written.  Token order: an
 * expert's n-th assignment in token order gets slot n.  Gate priority: slot
 * = rank by (gate descending, token ascending). */
int moe_dispatch(const moe_config *cfg, const void *x, const int32_t *expert_ids,
                 const float *gates, int32_t *slots, uint8_t *drop_mask,
                 int32_t *load, int32_t *kept, void *x_disp, void *ws,
                 size_t ws_bytes, void *stream);

/* Every expert's two-layer GELU FFN over its kept rows (survey notes sec.
 * 1.1.2.1; weight-only int8 dequantisation, survey notes sec. 1.2.3.1).
 * x_disp [E, C, d], kept [E] (device), w1/w2 (+ fp16 scales for int8).
 * Out: y_disp [E, C, d]; rows s >= kept[e] are not written.
 * Workspace: the hidden rows and, for int8 experts with C > 128 and
 * 32 <= E <= 256, a schedule of the experts over the XCDs computed on the
 * device from kept (16 E + 16 int32) that balances skewed expert loads. */
int moe_expert_ffn(const moe_config *cfg, const void *x_disp,
                   const int32_t *kept, const void *w1, const void *w1_scale,
                   const void *w2, const void *w2_scale, void *y_disp, void *ws,
                   size_t ws_bytes, void *stream);

/* PR-MoE's fixed dense MLP over all tokens ("DeepSpeed-MoE ... notes" sec.
 * 3.1): dense_out[t] = Wm2 GELU(Wm1 x[t]).  x [T, d]; out [T, d] act.
 * Workspace: moe_workspace_bytes(cfg, MOE_ENTRY_LAYER) covers it. */
int moe_dense_mlp(const moe_config *cfg, const void *x, const void *wm1,
                  const void *wm2, void *dense_out, void *ws, size_t ws_bytes,
                  void *stream);

/* Gate-weighted combine with residual ("DeepSpeed MoE and Model Compression",
 * combine(returned, gates); "DeepSpeed-MoE vs Switch Transformer", PR-MoE
 * residual example and overflow-through-residual):
 *   y[t] = base[t] + sum over j with slots[t,j] >= 0 of
 *          gates[t,j] * y_disp[expert_ids[t,j], slots[t,j]]
 * accumulated in fp32 in rank order j.  base [T, d] act or NULL (= 0);
 * base2 [T, d] act or NULL, added to base (x and D(x) for PR-MoE). */
int moe_combine(const moe_config *cfg, const void *y_disp,
                const int32_t *expert_ids, const int32_t *slots,
                const float *gates, const void *base, const void *base2,
                void *y, void *stream);

/* The whole layer: route, dispatch, [dense MLP], expert FFN, combine. */
int moe_layer_forward(const moe_config *cfg, const void *x,
                      const moe_weights *w, moe_outputs *out, void *ws,
                      size_t ws_bytes, void *stream);

/* moe_layer_forward without a workspace, for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc).  Same arguments, results and errors as
 * moe_layer_forward, except:
 *   - out->x_disp, out->y_disp and out->h_disp (each [E, C, *]) are required,
 *     and with pr_moe so are out->dense_out [T, d] and out->h_dense
 *     [T, d_ff_dense]: the caller owns every large buffer;
 *   - the remaining scratch (router partials, histograms, offsets, aux and
 *     z-loss partials, gate-priority segments, the int8 XCD schedule, the
 *     variant routers' scores) lives in the library's per-device array of
 *     MOE_NOALLOC_SCRATCH_BYTES; a configuration that needs more returns
 *     MOE_ERR_SCRATCH before anything is enqueued
 *     (moe_layer_forward_noalloc_scratch_bytes tells how much it needs);
 *   - the PR-MoE dense MLP runs in order on `stream` (overlap_dense is
 *     ignored: no side stream or event is created).
 * It calls no hipMalloc or hipFree and creates no stream or event (unless
 * moe_profile_enable is on).  Every call on one GPU uses that GPU's one
 * scratch array, which keeps the last call's contents: calls that overlap on
 * one GPU (concurrent streams or threads) race and must be serialised by the
 * caller; calls on different GPUs do not share it. */
int moe_layer_forward_noalloc(const moe_config *cfg, const void *x,
                              const moe_weights *w, moe_outputs *out,
                              void *stream);
/* Scratch bytes moe_layer_forward_noalloc needs for cfg (0 for an invalid
 * configuration); it runs when this is <= MOE_NOALLOC_SCRATCH_BYTES. */
size_t moe_layer_forward_noalloc_scratch_bytes(const moe_config *cfg);

/* Backward of moe_layer_forward: the gradients of
 *   <dy, y> + g_aux * aux_loss + g_z * z_loss
 * with respect to x and every weight, by the chain rule through the layer
 * ("DeepSpeed MoE and Model Compression", section DeepSpeed-MoE; a token
 * dropped by capacity skips the expert and gets no expert gradient,
 * "DeepSpeed-MoE vs Switch Transformer", section "expert capacity overflow";
 * the aux loss's f counts argmax decisions and is held constant; the top-k and
 * capacity decisions are held as the forward made them).
 * x, w: as given to the forward.  fwd: the forward's outputs for the same
 * cfg, x and w; expert_ids, gates, slots, logits, x_disp and y_disp are
 * required (so the forward must have been run with caller-owned logits,
 * x_disp and y_disp).  When the forward also kept z_disp and h_disp (and
 * z_dense and h_dense for PR-MoE), the backward reads them instead of
 * recomputing W1 x and GELU(W1 x).  dy [T, d] act.
 * Out: grads (written, not accumulated); the weight gradients are in the
 * activation type, accumulated in fp32.  bf16 activations, plain expert
 * weights and the softmax TopK router only (MOE_ERR_UNSUPPORTED otherwise).
 * Workspace:
 * moe_workspace_bytes(cfg, MOE_ENTRY_BACKWARD). */
int moe_layer_backward(const moe_config *cfg, const void *x, const moe_weights *w,
                       const moe_outputs *fwd, const void *dy, float g_aux, float g_z,
                       moe_grads *grads, void *ws, size_t ws_bytes, void *stream);

/* Rewrites one row-major bf16 expert weight tensor in MOE_W_BF16_PACKED
 * order, device to device, on `stream`: which = 1 packs W1 [E, d_ff, d],
 * which = 2 packs W2 [E, d, d_ff] (E, d, d_ff from cfg).  Both buffers are
 * the caller's, the same size, and must not overlap.  Meant to run once,
 * where the weights are loaded; the packed tensors then serve every forward
 * call with expert_wfmt = MOE_W_BF16_PACKED.
 * Errors: MOE_ERR_INVALID_ARG (null or misaligned pointer, which not 1 or 2,
 * an invalid cfg), MOE_ERR_UNSUPPORTED (fp32 activations, d or d_ff not a
 * multiple of 128). */
int moe_pack_expert_weights(const moe_config *cfg, int which, const void *w, void *w_packed,
                            void *stream);

/* Static description of a status code. */
const char *moe_status_string(int status);

/* Per-kernel timing (diagnostics).  When enabled, every kernel launch is
 * bracketed by a pair of HIP events recorded on its stream; moe_profile_read
 * synchronises those events and returns, per kernel name, the number of
 * launches and the summed duration in milliseconds since the last reset.
 * Not thread-safe; meant for one benchmarking thread. */
int moe_profile_enable(int on);
/* Restrict the timing records to launches whose name ("role:tile", as
 * moe_profile_read reports it) equals `name`; NULL or "" records every
 * launch.  Each record adds an event pair to its stream, so a benchmark that
 * times one kernel class keeps the others free of them. */
int moe_profile_filter(const char *name);
int moe_profile_reset(void);
/* Fills up to `cap` entries; returns the number of kernel names recorded. */
int moe_profile_read(char *names /* cap x 64 chars */, int64_t *launches,
                     double *total_ms, int cap);

#ifdef __cplusplus
}
#endif
#endif /* MOE_MI355X_H */
