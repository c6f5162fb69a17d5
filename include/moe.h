/* moe.h -- C ABI of libmoe: the forward pass of a group-limited top-k
 * sparse-MoE layer on one AMD Instinct MI355X (gfx950).
 *
 * The method is the one described on the page "InternLumina-U2中256个专家的路由
 * 秘密：分组受限Top-K、Expert Bias与Fused MoE详解" (cited [Routing §n], n its
 * numbered section):
 *   [Routing §二 step 1]  per-expert sigmoid scores of fp32 router logits;
 *   [Routing §二 step 2]  group-limited top-k: experts cut in index order into
 *                         n_group groups, group score = sum of the group's two
 *                         best scores, keep topk_group groups, top_k of those;
 *   [Routing §三]         expert_bias added to the scores for selection only;
 *   [Routing §二 step 3]  weights = unbiased scores / (their sum + 1e-20),
 *                         times routed_scaling_factor;
 *   [Routing §四]         stacked [E][I][H] SwiGLU experts;
 *   [Routing §五]         one shared expert added with no weight;
 *   [Routing §六]         per-expert hit counts (bincount of the choices).
 *
 * Conventions shared by every entry point
 *  - Pointers marked (device) are device memory of the current HIP device;
 *    (host) are host memory.  Arrays are row-major and contiguous; every
 *    device pointer must be 16-byte aligned (MOE_ERR_ALIGN otherwise).
 *  - Calls are asynchronous on `stream` and never synchronise, except
 *    moe_status.  The library keeps no pointer after a call returns and holds
 *    no mutable global state; concurrent calls on different workspaces are
 *    safe.  It allocates no memory: scratch space is the caller's workspace.
 *  - Results are deterministic: identical inputs give bit-identical outputs
 *    (no floating-point atomics anywhere).
 *  - Every error is detected on the host before anything is enqueued; on an
 *    error nothing is launched and no output is touched.  T = 0 is a no-op
 *    success.  Inputs are never written.  Outputs are fully overwritten,
 *    except `tracking`, which accumulates.
 *  - A selection tie goes to the lower group index, then to the lower expert
 *    index; the top_k chosen experts are returned in descending biased score.
 *  - sigma32, the router sigmoid, is specified exactly: the fp32 rounding
 *    (round to nearest even) of 1 / (1 + E(-z)) evaluated in IEEE fp64, where
 *    E(t) = 2^n * P(r), n = rint(t * RN(log2 e)), r = fma(-n, L2, fma(-n, L1, t))
 *    with L1 = RN(ln 2), L2 = RN(ln 2 - L1) (Cody & Waite reduction) and P the
 *    degree-13 Taylor polynomial of exp with coefficients RN(1/i!) by Horner
 *    fma; -z > 104 gives +0, -z < -40 gives 1, NaN gives NaN.
 */
#ifndef MOE_H
#define MOE_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ---- return codes -------------------------------------------------------- */
#define MOE_OK 0
#define MOE_ERR_INVALID (-1)     /* null required pointer, negative size, inconsistent shape */
#define MOE_ERR_UNSUPPORTED (-2) /* valid, but outside the kernels' envelope (see below) */
#define MOE_ERR_WORKSPACE (-3)   /* ws is NULL or ws_bytes < moe_workspace_size(desc) */
#define MOE_ERR_ALIGN (-4)       /* a device pointer is not 16-byte aligned */
#define MOE_ERR_HIP (-5)         /* a HIP call failed; moe_strerror gives no HIP code */
#define MOE_ERR_SCRATCH (-6)     /* moe_layer_forward_noalloc: the layer needs more scratch than
                                    MOE_NOALLOC_SCRATCH_BYTES */

/* ---- dtypes and flags ---------------------------------------------------- */
typedef enum { MOE_F32 = 0, MOE_BF16 = 1 } moe_dtype_t;

#define MOE_F_WRITE_LOGITS 1u /* moe_layer_forward writes logits_out (otherwise ignored) */
#define MOE_F_CHECK_FINITE 2u /* record non-finite router logits in the status word */

/* Status word bits, read by moe_status.  The first 256 bytes of a workspace
 * hold the status word: zero them before the workspace's first use. */
#define MOE_STATUS_NONFINITE 1u /* some token had a NaN/Inf router logit */
#define MOE_STATUS_BAD_INDEX 2u /* moe_permute met an index outside [0, E) (skipped) */

/* ---- layer description --------------------------------------------------- */
/* [Routing §一] gives the full-size values: E = 256, top_k = 8, n_group = 8,
 * topk_group = 4, one shared expert, I = 512, routed_scaling_factor = 2.5,
 * expert bias enabled; hidden size H = 2048.
 *
 * Envelope (MOE_ERR_UNSUPPORTED outside it): 2 <= E <= 512; E % n_group == 0;
 * group size E/n_group >= 2; n_group <= 64; 1 <= top_k <= 16;
 * top_k <= topk_group * E / n_group; H % 256 == 0 (bf16) or H % 64 == 0 and
 * H <= 16384 (fp32); I and I_shared multiples of 64 and at most 1024;
 * T < 2^30 and T * top_k < 2^31. */
typedef struct {
  int32_t T;                   /* tokens */
  int32_t H;                   /* hidden size */
  int32_t E;                   /* routed experts */
  int32_t n_group;             /* expert groups (contiguous index ranges) */
  int32_t topk_group;          /* groups kept per token */
  int32_t top_k;               /* experts chosen per token */
  int32_t I;                   /* routed expert intermediate size */
  int32_t I_shared;            /* shared expert intermediate size; 0 = no shared expert */
  float routed_scaling_factor; /* multiplies the normalised weights */
  int32_t dtype;               /* moe_dtype_t of x, y and all expert weights */
  uint32_t flags;              /* MOE_F_* */
} moe_desc_t;

/* Weights.  [Routing §四] stacks each projection of the E experts into one
 * tensor [E][I][H].  gate/up are used as z_i = sum_h x_h * W[e][i][h]; down,
 * stored [E][I][H] too, as out_h = sum_i a_i * W_down[e][i][h]. */
typedef struct {
  const float* w_router;    /* (device) [E][H] fp32 */
  const float* expert_bias; /* (device) [E] fp32, or NULL (= zeros) */
  const void* w_gate;       /* (device) [E][I][H] dtype */
  const void* w_up;         /* (device) [E][I][H] dtype */
  const void* w_down;       /* (device) [E][I][H] dtype */
  const void* ws_gate;      /* (device) [I_shared][H] dtype; NULL iff I_shared == 0 */
  const void* ws_up;        /* (device) [I_shared][H] dtype */
  const void* ws_down;      /* (device) [I_shared][H] dtype */
} moe_weights_t;

/* Bytes of device workspace every entry point below needs for `desc`
 * (one size covers all of them).  Host only.  Returns 0 on an invalid or
 * unsupported desc. */
size_t moe_workspace_size(const moe_desc_t* desc);

/* Router and selection [Routing §二 steps 1-3, §三].
 *   x           (device) [T][H] dtype
 *   w_router    (device) [E][H] fp32
 *   expert_bias (device) [E] fp32 or NULL
 *   logits      (device) [T][E] fp32, written when non-NULL: the fp32 router
 *               logits (the bf16 path computes them exactly as
 *               x . (hi + mid + lo) with W = hi + mid + lo split into three
 *               bf16 parts, fp32 accumulation)
 *   topk_idx    (device) [T][top_k] int32, descending biased score
 *   topk_w      (device) [T][top_k] fp32 routing weights
 * Tokens with a non-finite logit get topk_idx = 0..top_k-1 and topk_w = 0
 * (and the status bit when MOE_F_CHECK_FINITE is set). */
int moe_route(const moe_desc_t* desc, const void* x, const float* w_router,
              const float* expert_bias, float* logits, int32_t* topk_idx, float* topk_w,
              void* ws, size_t ws_bytes, hipStream_t stream);

/* Permute by expert [Routing §四 (inference buckets tokens by expert), §六].
 *   topk_idx    (device) [T][top_k] int32, each in [0, E); an index outside
 *               that range is skipped (not counted, pair_slot = -1) and sets
 *               MOE_STATUS_BAD_INDEX
 *   counts      (device) [E] int32: hits per expert
 *   offsets     (device) [E+1] int32: exclusive prefix sum, offsets[E] = T*top_k
 *   sorted_pair (device) [T*top_k] int32: pair ids p = t*top_k + j grouped by
 *               expert, ascending p inside each expert (stable)
 *   pair_slot   (device) [T*top_k] int32: inverse, sorted_pair[pair_slot[p]] = p
 *   tracking    (device) [E] int64 or NULL: tracking[e] += counts[e] */
int moe_permute(const moe_desc_t* desc, const int32_t* topk_idx, int32_t* counts,
                int32_t* offsets, int32_t* sorted_pair, int32_t* pair_slot, int64_t* tracking,
                void* ws, size_t ws_bytes, hipStream_t stream);

/* Experts and combine [Routing §四, §五]:
 *   y[t] = shared(x[t]) + sum_{j=0..top_k-1} topk_w[t][j] * expert_{e}(x[t])
 * with e the expert of pair t*top_k + j (from offsets/sorted_pair), the sum
 * taken in j order in fp32 and rounded once to dtype.  Inputs as produced by
 * moe_route / moe_permute; y (device) [T][H] dtype, must not alias x.
 * Hidden activations and per-pair outputs are rounded to dtype between the
 * projections. */
int moe_experts(const moe_desc_t* desc, const void* x, const float* topk_w,
                const int32_t* offsets, const int32_t* sorted_pair, const int32_t* pair_slot,
                const moe_weights_t* weights, void* y, void* ws, size_t ws_bytes,
                hipStream_t stream);

/* The whole layer: moe_route, moe_permute, moe_experts in sequence.  Every
 * *_out pointer may be NULL (then the workspace holds it); logits_out is only
 * written with MOE_F_WRITE_LOGITS.  tracking as in moe_permute. */
int moe_layer_forward(const moe_desc_t* desc, const void* x, const moe_weights_t* weights,
                      void* y, int32_t* topk_idx_out, float* topk_w_out, float* logits_out,
                      int32_t* counts_out, int64_t* tracking, void* ws, size_t ws_bytes,
                      hipStream_t stream);

/* For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): the same
 * layer forward as moe_layer_forward (the same kernels, bit-identical
 * results), with its workspace in a static buffer of the library instead of a
 * caller's `ws`.  The buffer is MOE_NOALLOC_SCRATCH_BYTES of device memory per
 * GPU, reserved by each GPU the library runs on until the process ends (it
 * holds the full-size layer, H 2048, I 512, at up to 512 tokens).  Nothing is
 * allocated: the first call on a device looks up that device's buffer address
 * once (the call's current device must be the stream's), and every call
 * clears the buffer's status word with a kernel before the layer's kernels.
 * All calls on one GPU share its buffer: calls that overlap in time on one GPU
 * (on different streams, or from different host threads) race and give
 * undefined results; serialise them.
 * Errors, on the host before anything is enqueued: those of moe_layer_forward
 * (a workspace error cannot occur); MOE_ERR_SCRATCH when
 * moe_workspace_size(desc) > MOE_NOALLOC_SCRATCH_BYTES; MOE_ERR_UNSUPPORTED
 * with MOE_F_CHECK_FINITE (the status word is not readable from outside). */
#define MOE_NOALLOC_SCRATCH_BYTES (32u << 20)
int moe_layer_forward_noalloc(const moe_desc_t* desc, const void* x, const moe_weights_t* weights,
                              void* y, int32_t* topk_idx_out, float* topk_w_out,
                              float* logits_out, int32_t* counts_out, int64_t* tracking,
                              hipStream_t stream);

/* Residual + RMSNorm for stacking layers (not on the pages; gamma = 1):
 *   x_out = RN(x_in + y)        (skipped, x_out = x_in, when y == NULL)
 *   r_out = RN(x_out / sqrt(mean(x_out^2) + eps))
 * all (device) [T][H] dtype, accumulation in fp32.  x_out may equal x_in. */
int moe_residual_rmsnorm(const moe_desc_t* desc, const void* x_in, const void* y, void* x_out,
                         void* r_out, float eps, hipStream_t stream);

/* Kernel stages of moe_layer_forward, in launch order (for measurement). */
typedef enum {
  MOE_STAGE_ROUTER_SPLIT = 0, /* bf16 only: router weight -> three bf16 parts */
  MOE_STAGE_LOGITS = 1,
  MOE_STAGE_SELECT = 2,
  MOE_STAGE_HIST = 3,
  MOE_STAGE_SCAN = 4,
  MOE_STAGE_SCATTER = 5,
  MOE_STAGE_TILES = 6,
  MOE_STAGE_GATE_UP = 7,
  MOE_STAGE_DOWN = 8,
  MOE_STAGE_COMBINE = 9,
  MOE_NUM_STAGES = 10
} moe_stage_t;

/* moe_layer_forward, plus: records `start` on `stream` immediately before the
 * kernel of `stage` is enqueued and `stop` immediately after, so that
 * hipEventElapsedTime(start, stop) is that kernel's duration.  Events are
 * caller-created; nothing else differs from moe_layer_forward.  For
 * measurement (a stage the desc does not launch records nothing). */
int moe_layer_forward_timed(const moe_desc_t* desc, const void* x, const moe_weights_t* weights,
                            void* y, int32_t* topk_idx_out, float* topk_w_out, float* logits_out,
                            int32_t* counts_out, int64_t* tracking, void* ws, size_t ws_bytes,
                            hipStream_t stream, int stage, hipEvent_t start, hipEvent_t stop);

/* Name of the kernel that moe_layer_forward launches for `stage` with this
 * desc, for the expert stages (MOE_STAGE_GATE_UP, _DOWN, _COMBINE), e.g.
 * "k_gateup_stream"; NULL for other stages or an invalid desc.  Host only; the
 * string is static.  For labelling measurements. */
const char* moe_stage_kernel(const moe_desc_t* desc, int stage);

/* Synchronises `stream`, then reads the workspace status word (MOE_STATUS_*)
 * into *status (host) and clears it. */
int moe_status(void* ws, size_t ws_bytes, hipStream_t stream, uint32_t* status);

/* The device implementation of sigma32 (see the header comment) applied to
 * z (device) [n] fp32 -> s (device) [n] fp32.  For verification. */
int moe_sigmoid32(const float* z, float* s, int64_t n, hipStream_t stream);

/* ---- load balancing -------------------------------------------------------
 * [Routing §六] keeps, per layer, a running count of each expert's hits (the
 * `tracking` that moe_permute / moe_layer_forward accumulate) and reads load
 * statistics from it; [Routing §三] moves the expert bias against each
 * expert's load during training (raised for experts that get few tokens,
 * lowered for those that get many); [Pitfalls, MoE 负载均衡 Loss 别忘加] adds
 * the load-balancing loss E * sum_i f_i * P_i.  These calls are small
 * reductions; they follow the conventions above (asynchronous, deterministic,
 * errors on the host before any launch, 16-byte aligned device pointers). */

#define MOE_NSTAT 8 /* summary values per layer of moe_expert_stats */

/* Load statistics of tracked hits, one row per layer.
 *   tracking (device) [L][E] int64 hits h[e] >= 0 (h[e] * E must fit int64)
 *   load     (device) [L][E] fp32: RN32(h[e] * E / N), N = sum_e h[e]; 1 is the
 *            balanced share; all 0 when N = 0
 *   summary  (device) [L][MOE_NSTAT] fp64: 0 N; 1 largest load; 2 smallest
 *            load; 3 coefficient of variation sqrt(mean_e (h[e] - N/E)^2) /
 *            (N/E); 4 experts with no hit; 5 most and 6 least hit expert
 *            (lower index on ties); 7 largest group load, (hits of the group,
 *            experts cut in index order into n_group groups) * n_group / N.
 *            With N = 0: entries 1, 2, 3, 7 are 0, 4 is E, 5 and 6 are 0.
 * Every value except entry 3 is exact as defined (one IEEE fp64 rounding per
 * operation shown); entry 3's sum runs in a fixed order of its own.
 * L = 0 is a no-op.  MOE_ERR_INVALID: L < 0, E < 1, E % n_group != 0, a null
 * pointer; MOE_ERR_UNSUPPORTED: E > 1024 or n_group > 64. */
int moe_expert_stats(int32_t L, int32_t E, int32_t n_group, const int64_t* tracking, float* load,
                     double* summary, hipStream_t stream);

/* Expert-bias update from one routing's hit counts ([Routing §三]; the page
 * gives no rule, this one moves each bias against its expert's hit excess
 * normalised by the largest excess).  In IEEE fp64:
 *   cbar = sum_e counts[e] / E,  d = max(max_e |counts[e] - cbar|, 1),
 *   bias_out[e] = RN32(bias_in[e] + (-rate * (counts[e] - cbar)) / d)
 *   counts   (device) [E] int32, e.g. moe_layer_forward's counts_out
 *   bias_in  (device) [E] fp32 or NULL (= zeros); bias_out (device) [E] fp32,
 *            may equal bias_in (update in place)
 * Results are bit-exact to the formula.  MOE_ERR_INVALID: E < 1, a null
 * required pointer, non-finite rate; MOE_ERR_UNSUPPORTED: E > 1024. */
int moe_bias_update(int32_t E, const int32_t* counts, const float* bias_in, float* bias_out,
                    double rate, hipStream_t stream);

/* Bytes of device workspace moe_aux_loss needs for T tokens and E experts
 * (0 if T < 1, T >= 2^30, E < 2 or E > 1024).  Host only. */
size_t moe_aux_loss_workspace_size(int32_t T, int32_t E);

/* Auxiliary load-balancing loss ([Pitfalls, MoE 负载均衡 Loss 别忘加]) from the
 * router logits the forward returns (MOE_F_WRITE_LOGITS) and the counts of
 * the routing taken, all in fp64:
 *   f[i] = counts[i] / T,  P[i] = (1/T) sum_t softmax(logits[t])[i],
 *   loss = E * sum_i f[i] * P[i]
 *   logits (device) [T][E] fp32; counts (device) [E] int32
 *   f, P   (device) [E] fp64; loss (device) [1] fp64
 *   ws     (device) moe_aux_loss_workspace_size(T, E) bytes of scratch
 * f is exact; P and loss carry fp64 rounding of the exponentials and of sums
 * taken in a fixed order (bit-reproducible).  A non-finite logit makes the
 * results non-finite.  MOE_ERR_INVALID: T < 1, E < 2, a null pointer;
 * MOE_ERR_UNSUPPORTED: E > 1024 or T >= 2^30; MOE_ERR_WORKSPACE: ws too small. */
int moe_aux_loss(int32_t T, int32_t E, const float* logits, const int32_t* counts, double* f,
                 double* P, double* loss, void* ws, size_t ws_bytes, hipStream_t stream);

/* ---- backward ---------------------------------------------------------------
 * The layer's backward for the routing the forward chose (the training
 * context of [Pitfalls]): the chosen experts are held fixed (the choice is
 * piecewise constant; the expert bias only enters the choice, so it gets no
 * gradient), the routing weights w_j = scale * s_j / (sum_k s_k + 1e-20) are
 * differentiated through the sigmoid scores s = sigmoid(logit) of the chosen
 * experts ([Routing §二 steps 1-3]), and y = shared(x) + sum_j w_j expert_j(x)
 * ([Routing §四, §五]) through both projections of every SwiGLU expert.
 * Envelope: as the forward, plus dtype MOE_BF16 and I_shared == 0 or == I
 * (MOE_ERR_UNSUPPORTED otherwise). */

/* Bytes of device workspace moe_layer_backward needs (0 on an invalid or
 * unsupported desc).  Host only. */
size_t moe_backward_workspace_size(const moe_desc_t* desc);

/* Gradients of L = sum dy * y for the layer of `desc`:
 *   x, weights   the forward's inputs (w_router and the expert weights are
 *                read; expert_bias is not used)
 *   topk_idx     (device) [T][top_k] int32: the chosen experts (the forward's
 *                topk_idx_out), each in [0, E) (an index outside it gives
 *                unspecified gradients for its token; every access stays
 *                in bounds)
 *   logits       (device) [T][E] fp32: router logits (the forward's
 *                logits_out with MOE_F_WRITE_LOGITS)
 *   dy           (device) [T][H] bf16: upstream gradient of y
 *   dx           (device) [T][H] bf16 (out; must not alias x or dy)
 *   dw_router    (device) [E][H] fp32 (out)
 *   dw_gate, dw_up, dw_down    (device) [E][I][H] fp32 (out; zero for
 *                experts no token chose)
 *   dws_gate, dws_up, dws_down (device) [I_shared][H] fp32 (out), NULL iff
 *                I_shared == 0
 * Intermediates (g, u, r = dy W_down^T, the activation gradients) are bf16
 * MFMA operands or fp32; accumulation is fp32; every sum runs in a fixed
 * order (bit-reproducible).  T = 0 is a no-op. */
int moe_layer_backward(const moe_desc_t* desc, const void* x, const moe_weights_t* weights,
                       const int32_t* topk_idx, const float* logits, const void* dy, void* dx,
                       float* dw_router, float* dw_gate, float* dw_up, float* dw_down,
                       float* dws_gate, float* dws_up, float* dws_down, void* ws,
                       size_t ws_bytes, hipStream_t stream);

/* Static description of an error code. */
const char* moe_strerror(int code);

#ifdef __cplusplus
}
#endif
#endif /* MOE_H */
