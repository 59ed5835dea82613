/*
 * moe.h — C ABI of the MI355X (gfx950) sparse Mixture-of-Experts FFN layer forward.
 *
 * The layer (kwkr.cn page on sparse activation, news/623730, sections 2.1-2.3 and 3.1-3.2):
 *   1. router:   z = x W_g^T (+ b_g), float32 logits; scores s = (z + g) / tau, with g the
 *                Gumbel noise of the Gumbel-softmax router ("Mixture of Experts (MoE)
 *                原理与工程落地全指南", lpnh.cn, section 2.2) when enabled, else s = z / tau;
 *                p = softmax(s) in float32.
 *   2. top-k:    the k largest scores per token, largest first, lower expert index first on
 *                equal scores; weights w_j = p[idx_j] / sum_j' p[idx_j'] (sum to 1).
 *   3. dispatch: C = ceil(c k T / E); slots (t, j) taken in token order; each expert keeps its
 *                first C slots, later ones are dropped (contribute zero).
 *   4. experts:  H = GeLU(x_e W1_e^T + b1_e) (exact erf GeLU), y_e = H W2_e^T + b2_e, run only on
 *                each expert's own kept rows.
 *   5. combine:  y[t] = sum over kept j of w[t,j] * y_e[t]; and the balance statistic
 *                f_e = counts_e / (k T), P_e = mean_t p[t,e], L = E sum_e f_e P_e.
 *
 * Conventions for every entry point:
 *   - Tensor pointers are DEVICE pointers, row-major and contiguous, owned by the caller.
 *     Weights use nn.Linear's [out, in] layout: W_g [E,d], W1 [E,d_ffn,d], W2 [E,d,d_ffn].
 *   - "dtype" tensors (x, W_g, W1, b1, W2, b2, x_perm, y) are bfloat16 or float32 per
 *     moe_config.dtype; b_g, logits, scores, weights, y_perm and statistics are float32;
 *     indices and counts are int32.
 *   - Alignment: dtype and float tensors 16 bytes, int32 arrays 4 bytes, the workspace 256
 *     bytes. Optional (nullable) pointers are marked.
 *   - Every call is asynchronous on `stream` (NULL = the default stream) and does no host
 *     synchronisation; results are valid once the caller synchronises the stream. The
 *     library allocates nothing and keeps no state between calls.
 *   - Arguments are validated before anything is enqueued; on any error nothing is enqueued
 *     and a status is returned (never printed, never aborted). Detail: moe_last_error().
 *   - Rows of the expert-sorted buffers (x_perm, y_perm, perm) beyond sum(kept) are left
 *     untouched.
 *   - Results are deterministic: no floating-point atomics; every sum has a fixed order.
 */
#ifndef MOE_H
#define MOE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Opaque handles; these are hipStream_t and hipEvent_t. */
typedef struct ihipStream_t* moe_stream_t;
typedef struct ihipEvent_t* moe_event_t;

typedef enum {
  MOE_OK = 0,
  MOE_EINVAL = 1,        /* null required pointer, bad size, k > E, c or tau <= 0 / not finite,
                            misaligned pointer, k*T >= 2^31 */
  MOE_EUNSUPPORTED = 2,  /* E > 64, k > 8, bf16 with d or d_ffn not a multiple of 64, float32
                            beyond its size limits, c > 2^20 */
  MOE_EWORKSPACE = 3,    /* workspace smaller than moe_workspace_size() */
  MOE_EHIP = 4           /* a HIP launch error; text in moe_last_error() */
} moe_status;

typedef enum { MOE_F32 = 0, MOE_BF16 = 1 } moe_dtype;

/* Layer configuration (kwkr.cn page, section 2: T tokens, d model dim, E experts, top-k,
 * capacity factor c; section 3.1: expert hidden width d_ffn). */
typedef struct moe_config {
  int64_t T;               /* tokens (a [B,S,d] batch flattened to [T,d]; t = b*S + s)      */
  int64_t d;               /* model dimension                                              */
  int64_t E;               /* experts, 1..64                                               */
  int64_t k;               /* experts per token, 1..min(E, 8)                              */
  int64_t d_ffn;           /* expert hidden dimension                                      */
  double capacity_factor;  /* c > 0; C = ceil(c*k*T/E) from the exact value of this double */
  float temperature;       /* tau > 0; 1 = plain softmax                                   */
  int32_t gumbel;          /* 0: s = z/tau. 1: s = (z + g)/tau, g = -log(-log u) with u from
                              Philox-4x32-10, key = (seed mod 2^32, seed >> 32),
                              counter = (t, e, 0, 0), u = (word0 + 1/2) 2^-32, computed in
                              float64 and rounded once to float32                          */
  uint64_t seed;           /* Philox key when gumbel = 1                                    */
  int32_t dtype;           /* moe_dtype: storage of x, weights, x_perm, H and y            */
  int32_t reserved;        /* must be 0                                                    */
} moe_config;

/* Number of kernel stages of moe_forward (route, scan, permute+gather, expert GEMM1+GeLU,
 * expert GEMM2, combine); moe_forward_aux.stage_events takes MOE_FORWARD_STAGES + 1 events.
 * Under token-order dropping the permutation is recorded in the scan stage (for batches of at
 * most 1024 tokens it runs inside the scan kernel), so the third stage holds only the gather,
 * which the bf16 expert paths usually fuse into their operand loads: it can be empty. */
#define MOE_FORWARD_STAGES 6

/* Optional extra outputs of moe_forward. Every pointer may be NULL. */
typedef struct moe_forward_aux {
  float* logits;           /* [T,E] float32 z                                               */
  float* scores;           /* [T,E] float32 s (equal to the logits when gumbel = 0, tau = 1) */
  int32_t* topk_idx;       /* [T,k]                                                         */
  float* topk_w;           /* [T,k]                                                         */
  int32_t* offsets;        /* [E] exclusive prefix sum of kept                              */
  int32_t* dest;           /* [T,k] row of slot (t,j) in the expert-sorted buffer, -1 = dropped */
  int32_t* perm;           /* [min(k*T, E*C)] source token of each expert-sorted row        */
  float* prob_colsum;      /* [E] sum_t p[t,e]                                              */
  moe_event_t* stage_events; /* NULL, or MOE_FORWARD_STAGES+1 created events, recorded on
                                `stream` before each stage and after the last              */
} moe_forward_aux;

/* C = ceil(c*k*T/E) (kwkr.cn page, section 2.3), exact integer arithmetic on the double c.
 * Host only. Returns -1 when the configuration is invalid. */
int64_t moe_capacity(const moe_config* cfg);

/* Workspace bytes that every entry point below needs for `cfg` (the largest is moe_forward's:
 * per-block partial sums and histograms, routing arrays, x_perm, H and y_perm). Host only. */
moe_status moe_workspace_size(const moe_config* cfg, size_t* bytes);

/* Router: steps 1-2 (kwkr.cn page, section 2.1; lpnh.cn page, section 2.2).
 *   x [T,d] dtype, Wg [E,d] dtype, bg [E] float32 (nullable)
 *   -> logits [T,E] f32; scores [T,E] f32 (nullable; written when non-NULL);
 *      topk_idx [T,k] i32; topk_w [T,k] f32; prob_colsum [E] f32 = sum_t p[t,e]. */
moe_status moe_route(const moe_config* cfg, const void* x, const void* Wg, const float* bg,
                     float* logits, float* scores, int32_t* topk_idx, float* topk_w,
                     float* prob_colsum, void* ws, size_t ws_bytes, moe_stream_t stream);

/* Dispatch: step 3 (kwkr.cn page, sections 2.3 and 3.2): per-expert histogram, prefix scan,
 * capacity truncation and the stable permutation, then the row gather x_perm[r] = x[perm[r]].
 *   topk_idx [T,k] i32 (each row k distinct experts in [0,E)), x [T,d] dtype
 *   -> counts, kept, offsets [E] i32; dest [T,k] i32 (-1 = dropped);
 *      perm [min(k*T, E*C)] i32; x_perm [min(k*T, E*C), d] dtype. */
moe_status moe_dispatch(const moe_config* cfg, const int32_t* topk_idx, const void* x,
                        int32_t* counts, int32_t* kept, int32_t* offsets, int32_t* dest,
                        int32_t* perm, void* x_perm, void* ws, size_t ws_bytes,
                        moe_stream_t stream);

/* Experts: step 4 (kwkr.cn page, section 3.1; intelliparadigm.com page, section 2.1):
 * rows [offsets[e], offsets[e]+kept[e]) of x_perm go through expert e.
 *   x_perm [R,d] dtype, kept/offsets [E] i32 (as moe_dispatch writes them),
 *   W1 [E,d_ffn,d], b1 [E,d_ffn] (nullable), W2 [E,d,d_ffn], b2 [E,d] (nullable), all dtype
 *   -> y_perm [R,d] f32. H [R,d_ffn] lives in the workspace. */
moe_status moe_expert_ffn(const moe_config* cfg, const void* x_perm, const int32_t* kept,
                          const int32_t* offsets, const void* W1, const void* b1, const void* W2,
                          const void* b2, float* y_perm, void* ws, size_t ws_bytes,
                          moe_stream_t stream);

/* Combine and statistics: step 5 (kwkr.cn page, sections 2.1, 2.2 and 3.2; intelliparadigm.com
 * page, section 2.3). y[t] = sum_j w[t,j] * y_perm[dest[t,j]] over kept slots, in j order, in
 * float32, rounded once to dtype; a token whose slots were all dropped gets y = 0.
 *   y_perm [R,d] f32, dest [T,k] i32, topk_w [T,k] f32, counts [E] i32, prob_colsum [E] f32
 *   -> y [T,d] dtype; f [E], P [E], L [1] f32 (f, P, L nullable together). */
moe_status moe_combine(const moe_config* cfg, const float* y_perm, const int32_t* dest,
                       const float* topk_w, const int32_t* counts, const float* prob_colsum,
                       void* y, float* f, float* P, float* L, void* ws, size_t ws_bytes,
                       moe_stream_t stream);

/* The whole layer, steps 1-5, on one stream with no host synchronisation.
 *   x, Wg, bg, W1, b1, W2, b2 as above -> y [T,d] dtype; f, P [E] f32; L [1] f32;
 *   counts, kept [E] i32; aux (nullable) for the intermediate results and stage timing. */
moe_status moe_forward(const moe_config* cfg, const void* x, const void* Wg, const float* bg,
                       const void* W1, const void* b1, const void* W2, const void* b2,
                       void* y, float* f, float* P, float* L, int32_t* counts, int32_t* kept,
                       const moe_forward_aux* aux, void* ws, size_t ws_bytes,
                       moe_stream_t stream);

/* moe_forward for callers that cannot allocate device memory (code under HIP graph capture,
 * tight serving loops, harnesses that forbid hipMalloc): the workspace is a static device
 * array of MOE_NOALLOC_SCRATCH_BYTES inside the library instead of the caller's ws. Arguments
 * and results as moe_forward; the caller still passes every input and output buffer.
 *   - Uses the scratch of the calling thread's current device; `stream` must belong to it.
 *     The first call on a device looks the array's address up there (no allocation); every
 *     GPU the library runs on holds the array until the process ends.
 *   - Every call on one GPU shares that GPU's array: calls that overlap on one GPU (other
 *     streams, other threads) race and must be serialised by the caller. Nothing in the
 *     array needs to start at zero; it keeps the last call's intermediates.
 *   - Calls no hipMalloc, hipFree or allocating library routine.
 *   - MOE_EUNSUPPORTED when moe_workspace_size(cfg) exceeds MOE_NOALLOC_SCRATCH_BYTES
 *     (decode-sized batches and small layers fit; the named large layers do not), checked
 *     before any HIP call; other errors as moe_forward. */
#define MOE_NOALLOC_SCRATCH_BYTES (64u << 20)
moe_status moe_forward_noalloc(const moe_config* cfg, const void* x, const void* Wg, const float* bg,
                               const void* W1, const void* b1, const void* W2, const void* b2,
                               void* y, float* f, float* P, float* L, int32_t* counts, int32_t* kept,
                               const moe_forward_aux* aux, moe_stream_t stream);

/* ---------------------------------------------------------------------------------------
 * Forward variants. A zeroed moe_variant is the plain layer above, and moe_forward_ex with
 * variant = NULL is moe_forward. Stage calls (moe_route ... moe_combine) take no variant.
 */
typedef enum { MOE_ACT_GELU = 0, MOE_ACT_SILU = 1 } moe_activation;

/* What happens to the slots past an expert's capacity C (mhpn.cn page on MoE architecture,
 * section 3.3, names dropping at random and rerouting to the next-best expert besides the
 * first-come order of the kwkr.cn page, sections 2.3 and 3.2). */
typedef enum {
  MOE_DROP_TOKEN_ORDER = 0, /* keep the first C slots in token order (the plain layer)        */
  MOE_DROP_RANDOM = 1,      /* keep the C slots with the smallest (priority, token), priority =
                               word 2 of the Philox-4x32-10 block of counter (t, e, 0, 0) under
                               the config's seed (words 0 and 1 feed the router noise); the
                               kept rows of an expert stay in token order                    */
  MOE_DROP_REROUTE = 2      /* pass 1 is token order; a token's slots dropped there take, in j
                               order, its (k+1)-th, (k+2)-th ... ranked experts (by score,
                               lower index on ties; none past the E-th), and pass 2 fills the
                               capacity left after pass 1 in slot order (t k + j). An expert's
                               rows are its pass-1 rows, then its pass-2 rows. A token with a
                               moved slot has its weights renormalised over the experts its
                               slots end at: w_j = p_{e_j} / sum_j' p_{e_j'}, computed as
                               exp(s_j - m) / sum exp(s_j' - m) from the float32 scores.
                               counts, f, P, L are those of pass 1; kept is final;
                               aux.topk_idx holds the pass-1 choices, aux.topk_w the final
                               weights                                                         */
} moe_drop_policy;

/* Storage of W1 and W2 (the routed experts' weights; a shared expert's stay row-major). */
typedef enum {
  MOE_WEIGHTS_LINEAR = 0,   /* nn.Linear's row-major [E,d_ffn,d] and [E,d,d_ffn]                */
  MOE_WEIGHTS_PACKED = 1    /* the same bytes reordered by moe_pack_expert_weights: a layout for
                               serving, packed once when the weights are loaded. bf16 only, d
                               and d_ffn multiples of 256; the results are bit-identical to the
                               row-major layout's. Not taken by the training entry points.     */
} moe_weight_layout;

/* Number of floats moe_variant.route_stats receives. */
#define MOE_ROUTE_STATS 5

typedef struct moe_variant {
  int32_t activation;      /* moe_activation of every expert (routed and shared): GeLU, or
                              SiLU(v) = v sigmoid(v) (lpnh.cn page, section 3.2)            */
  float noise_std;         /* 0: no Gaussian noise. > 0 (needs gumbel = 0): s = (z + g)/tau,
                              g = noise_std * n with n standard normal per (token, expert)
                              (kwkr.cn page, section 3.3): from the Philox block of the Gumbel
                              noise (same key, counter (t, e, 0, 0)), u1 and u2 = (word 0 or
                              word 1 + 1/2) 2^-32, n = sqrt(-2 ln u1) cos(2 pi u2) in float64,
                              and g = noise_std * n rounded once to float32                 */
  int64_t shared_d_ffn;    /* 0: none. Else the hidden width of one shared expert that every
                              token uses (lpnh.cn page, section 2.3):
                              y[t] = FFN_s(x[t]) + sum_j w[t,j] FFN_e(x[t]); the float32 sum
                              starts from FFN_s and adds the slots in j order. bf16 needs a
                              multiple of 64.                                                 */
  const void* W1s;         /* [shared_d_ffn, d] dtype (required when shared_d_ffn > 0)        */
  const void* b1s;         /* [shared_d_ffn] dtype, nullable                                  */
  const void* W2s;         /* [d, shared_d_ffn] dtype (required when shared_d_ffn > 0)        */
  const void* b2s;         /* [d] dtype, nullable                                             */
  int32_t drop_policy;     /* moe_drop_policy                                                 */
  int32_t weight_layout;   /* moe_weight_layout of W1 and W2                                    */
  float* route_stats;      /* nullable; else [MOE_ROUTE_STATS] f32 on the device, written by the
                              layer from the counts before capacity (u_e = counts_e / T) and
                              the full softmax p, each in float64 rounded once to float32
                              (lpnh.cn page, sections 2.4 and 3.6; mhpn.cn page, 3.1):
                              [0] sum_e u_e^2; [1] 0.5 Q50 + 0.3 Q90 + 0.2 Q99 of u, Qq by
                              linear interpolation at position (E-1) q of the sorted u;
                              [2] sum_e (counts_e - mean counts)^2; [3] population standard
                              deviation of u; [4] mean over tokens of -sum_e p ln p (0 ln 0 =
                              0; per-token terms in float32, summed in a fixed order)         */
} moe_variant;

/* Workspace bytes of moe_forward_ex for `cfg` and `variant` (nullable). Host only.
 * MOE_EINVAL for an unknown activation or drop policy, a negative or non-finite noise_std,
 * noise_std > 0 together with gumbel = 1, an unknown weight_layout, or a misaligned
 * route_stats; MOE_EUNSUPPORTED for a shared_d_ffn the dtype cannot take, or packed weights
 * with float32, or d or d_ffn not a multiple of 256. */
moe_status moe_workspace_size_ex(const moe_config* cfg, const moe_variant* variant, size_t* bytes);

/* The layer with the variant's activation, router noise and shared expert; arguments as
 * moe_forward. With a shared expert, stage 5 of aux.stage_events (expert GEMM2) also covers
 * the shared expert's two GEMMs. */
moe_status moe_forward_ex(const moe_config* cfg, const moe_variant* variant, const void* x,
                          const void* Wg, const float* bg, const void* W1, const void* b1,
                          const void* W2, const void* b2, void* y, float* f, float* P, float* L,
                          int32_t* counts, int32_t* kept, const moe_forward_aux* aux, void* ws,
                          size_t ws_bytes, moe_stream_t stream);

/* Packs one expert weight tensor for variant.weight_layout = MOE_WEIGHTS_PACKED: W [E,rows,cols]
 * row-major bf16 (W1 with rows = d_ffn, cols = d; W2 with rows = d, cols = d_ffn) -> W_packed,
 * E*rows*cols bf16 values in panels: panel e*(rows/256) + p holds rows [256 p, 256 p + 256) of
 * expert e as cols/32 consecutive blocks of 256 rows x 32 columns, each row of a block the 64
 * contiguous bytes of its 32 values. The expert GEMMs then load each K step of a 256-row tile
 * as one contiguous 16 KB block (whole cache lines) instead of 256 half lines. Pure data
 * movement, no rounding. Both pointers are device pointers, 16-byte aligned, caller-owned and
 * must not overlap. Asynchronous on `stream`.
 * MOE_EINVAL: a NULL or misaligned pointer, overlapping buffers, E < 1, rows < 1, cols < 1, any
 * of them above 2^20, or E*rows*cols above 2^40;
 * MOE_EUNSUPPORTED: rows not a multiple of 256 or cols not a multiple of 32; MOE_EHIP: the
 * launch failed. */
moe_status moe_pack_expert_weights(int64_t E, int64_t rows, int64_t cols, const void* W, void* W_packed,
                                   moe_stream_t stream);

/* ---------------------------------------------------------------------------------------
 * Backward pass (kwkr.cn page on sparse activation, sections 2.2, 2.3 and 3.3): the gradients
 * of J = sum(dy * y) + lam * L. The routing decisions (top-k, capacity, the drop policy) and
 * f are discrete and carry no gradient; the combine weights w and the balance term's P do. A
 * dropped slot contributes nothing to y, but its probability stays in its token's
 * renormalisation, so it still reaches the router:
 *   dw_tj = <dy_t, FFN_e(x_t)> (kept slots), w_tj = p_t,e_j / sum_j' p_t,e_j' over the token's
 *   k final experts, dP_e = lam E f_e / T per token, softmax and 1/tau back to the logits;
 *   expert e: dW2 = sum (w dy)^T h, dW1 = sum dA^T x with dA = (w dy W2_e) * act'(a); dx gets
 *   dA W1_e per kept slot and dz W_g; the noise is a constant.
 * Precision: bf16 storage keeps the pre-activations a and the products dA and w dy in bf16
 * (MFMA operands) with float32 accumulation; float32 storage computes in float32. A shared
 * expert is not covered (MOE_EUNSUPPORTED). */

/* Stages of moe_backward (router backward, weight transposes, dA product, dx product, row
 * transposes, dW2 product, dW1 product, bias / router / input gradients). */
#define MOE_BACKWARD_STAGES 8

typedef struct moe_backward_aux {
  float* dz;                 /* NULL, or [T,E] f32: receives the logit gradient                */
  moe_event_t* stage_events; /* NULL, or MOE_BACKWARD_STAGES+1 created events                  */
} moe_backward_aux;

/* Workspace bytes of moe_forward_train + moe_backward for cfg and variant (nullable). This
 * includes the saved state (pre-activations [R, d_ffn], routing, expert outputs) and the
 * backward's scratch (the transposed weights: 2 E d d_ffn elements). Host only. */
moe_status moe_workspace_size_train(const moe_config* cfg, const moe_variant* variant, size_t* bytes);

/* moe_forward_ex that also keeps in ws everything moe_backward needs. The routing arrays stay
 * in ws; aux pointers, when given, receive copies. Same arguments and outputs. */
moe_status moe_forward_train(const moe_config* cfg, const moe_variant* variant, const void* x,
                             const void* Wg, const float* bg, const void* W1, const void* b1,
                             const void* W2, const void* b2, void* y, float* f, float* P, float* L,
                             int32_t* counts, int32_t* kept, const moe_forward_aux* aux, void* ws,
                             size_t ws_bytes, moe_stream_t stream);

/* Gradients after moe_forward_train with the same cfg, variant, inputs and ws (unchanged in
 * between). dy [T,d] dtype; lam: the weight of L in J.
 *   dx [T,d] dtype; dWg [E,d] f32; dbg [E] f32 (nullable); dW1 [E,d_ffn,d] f32; db1 [E,d_ffn]
 *   f32 (nullable); dW2 [E,d,d_ffn] f32; db2 [E,d] f32 (nullable). Experts without kept rows
 *   get zero weight gradients. Every sum has a fixed order (bitwise reproducible). */
moe_status moe_backward(const moe_config* cfg, const moe_variant* variant, const void* x,
                        const void* Wg, const void* W1, const void* W2, const void* dy, float lam,
                        void* dx, float* dWg, float* dbg, float* dW1, float* db1, float* dW2,
                        float* db2, const moe_backward_aux* aux, void* ws, size_t ws_bytes,
                        moe_stream_t stream);

/* Temperature schedule tau_t = max(tau_min, tau0 - rate * step) (lpnh.cn page, section 3.3:
 * tau0 = 1, tau_min = 0.5, rate = 1e-4; aberweb.com page, section 3.3: rate 1e-3), computed in double and
 * rounded once to float; the result goes to moe_config.temperature. Host only. */
float moe_temperature_at(int64_t step, float tau0, float tau_min, float rate);

/* Static text of a status code. */
const char* moe_status_str(moe_status status);

/* Detail of the last non-OK return on the calling thread ("" if none). */
const char* moe_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* MOE_H */
