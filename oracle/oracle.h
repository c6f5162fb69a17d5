/* oracle.h -- TEST INFRASTRUCTURE ONLY.
 *
 * Plain, slow CPU reference of the forward pass of a group-limited top-k
 * sparse-MoE layer (sigmoid router, expert bias for selection only, 256
 * stacked SwiGLU experts plus one shared expert, weighted combine).  Only the
 * test-suite, the smoke check and the CPU-baseline leg of the benchmark may
 * load it.  It shares no code, header, table or constant with the HIP library
 * it checks.
 *
 * Source of the method: the page "InternLumina-U2中256个专家的路由秘密：分组受限
 * Top-K、Expert Bias与Fused MoE详解" (yfxerp.com/news/374153), cited below as
 * [Routing §n] with n the page's own numbered section (一..七).  The page at
 * m.lqnn.cn/news/279712 is cited as [Pitfalls, <section heading>].
 *
 * All pointers are host pointers to row-major, contiguous arrays.  Activation
 * and expert-weight arrays are either fp32 (ORC_F32) or bf16 stored as raw
 * uint16 bit patterns (ORC_BF16); every element is widened exactly to double
 * before use.  Floating-point results are fp64 unless stated.
 */
#ifndef MOE_ORACLE_H
#define MOE_ORACLE_H
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum { ORC_F32 = 0, ORC_BF16 = 1, ORC_F64 = 2 };

/* sigma32: the fp32 logistic function as specified in oracle.c (fp64 Cody-Waite
 * exp + degree-13 Taylor, one division, one rounding to fp32). */
float orc_sigmoid32(float z);
void orc_sigmoid32_array(const float* z, float* s, int64_t n);

/* Accuracy/monotonicity scan of sigma32 over the fp32 bit patterns
 * start, start+stride, ... < stop (as uint64 to allow stop = 2^32).
 * out[0] = inputs checked, out[1] = results != RN32(long-double reference),
 * out[2] = results more than 1 ulp from the reference, out[3] = monotonicity
 * violations between consecutive checked inputs of equal sign. */
void orc_sigmoid32_scan(uint64_t start, uint64_t stop, uint64_t stride, int nthreads,
                        int64_t out[4]);

/* sigma32 of the n fp32 bit patterns start .. start + n - 1 compared with
 * other[0 .. n-1] (another implementation's results for the same patterns):
 * out[0] = patterns whose results differ (bits differ and not both NaN),
 * out[1] = index of the first such pattern, or -1. */
void orc_sigmoid32_compare(uint64_t start, uint64_t n, const float* other, int nthreads,
                           int64_t out[2]);

/* R1: router logits l[t][e] = sum_h x[t][h]*w_router[e][h] in fp64. */
void orc_logits(int T, int H, int E, const void* x, int xdt, const float* w_router,
                double* logits, int nthreads);

/* R2..R8: selection from fp32 logits lam[T][E].  bias may be NULL.
 * Writes idx[T][K] (int32), w[T][K] (fp32) and flag[T] (1 = a non-finite
 * logit; that row's idx/w are then set to -1 / 0).  Returns the number of
 * flagged tokens, or -1 on an invalid shape. */
int orc_select(int T, int E, int n_group, int topk_group, int K, float scale,
               const float* lam, const float* bias, int32_t* idx, float* w, uint8_t* flag);

/* Interval analysis used to decide which tokens have a unique selection when
 * every fp32 logit may sit anywhere in [l - tau, l + tau] (l = fp64 logit,
 * tau = tau_abs + tau_rel * |l|).
 * Writes per token: decided[t] bit0 = set of K experts unique, bit1 = also
 * their order unique; and the bounds sb_lo/sb_hi [T][E], gs_lo/gs_hi
 * [T][n_group] (fp32).  Any output pointer except decided may be NULL. */
int orc_route_intervals(int T, int E, int n_group, int topk_group, int K,
                        const double* logits, double tau_abs, double tau_rel, const float* bias,
                        const int32_t* idx_ref, uint8_t* decided, float* sb_lo,
                        float* sb_hi, float* gs_lo, float* gs_hi);

/* a5: counts, exclusive offsets[E+1], stable counting sort of pair ids
 * p = t*K + j by expert, and its inverse. */
void orc_permute(int T, int K, int E, const int32_t* idx, int32_t* counts, int32_t* offsets,
                 int32_t* sorted_pair, int32_t* pair_slot);

typedef struct {
  int H, I, I_shared, E, K;
  int wdt;                        /* ORC_F32 or ORC_BF16 for all expert weights */
  const void *w_gate, *w_up, *w_down;        /* [E][I][H] each */
  const void *ws_gate, *ws_up, *ws_down;     /* [I_shared][H] each, or NULL */
} orc_experts_t;

/* a6..a8, path A: per token, per routed slot j, the SwiGLU expert in fp64,
 * then y = shared + sum_j w_j * out_j in j order.  Computes the rows
 * tokens[0..n_tok) (or 0..n_tok when tokens == NULL) into y[n_tok][H]. */
void orc_experts_path_a(const orc_experts_t* ex, const void* x, int xdt, const int32_t* idx,
                        const float* w, const int32_t* tokens, int n_tok, double* y, int nthreads);

/* a6..a8, path B: bucket the T*K pairs by expert with orc_permute, run each
 * bucket through its expert into a per-pair buffer, then combine in j order.
 * Computes all T rows. */
void orc_experts_path_b(const orc_experts_t* ex, int T, const void* x, int xdt,
                        const int32_t* idx, const float* w, double* y, int nthreads);

/* a9 (layer stack only): r = x / sqrt(mean(x^2) + eps), gamma = 1, fp64. */
void orc_rmsnorm(int T, int H, const void* x, int xdt, double eps, double* r);

/* Load balancing ([Routing §三, §六], [Pitfalls, MoE 负载均衡 Loss 别忘加]);
 * definitions in oracle.c. */
enum { ORC_NSTAT = 8 };
void orc_track(int T, int K, int E, const int32_t* idx, int64_t* tracking);
void orc_expert_stats(int L, int E, int n_group, const int64_t* tracking, float* load,
                      double* summary);
void orc_bias_update(int E, const int32_t* counts, const float* bias_in, float* bias_out,
                     double rate);
void orc_aux_loss(int T, int E, const float* lam, const int32_t* counts, double* f, double* P,
                  double* loss);

/* Backward of the layer for a fixed routing (definitions and the chain rule
 * in oracle.c), fp64 with the exact logistic sigmoid.  lam [T][E] are the
 * fp64 router logits; dy [T][H] the upstream gradient.
 * orc_backward_tokens: for the rows tokens[0..n_tok) (all T when NULL):
 *   dx [n_tok][H], dweight [n_tok][K] (dL/dw_j), dlogit [n_tok][E] (dL/dlam,
 *   zero off the chosen experts) and, if y != NULL, the fixed-routing forward
 *   y [n_tok][H]; any output may be NULL.
 * orc_backward_expert_weights: dW_gate, dW_up, dW_down of expert e (e == E:
 *   the shared expert), each [I][H] (I_shared for the shared expert).
 * orc_router_weight_grad: dW_r [E][H] from dlogit [T][E].
 * orc_logits_any: lam = x . W_r^T in fp64 (x, W_r of any ORC_ dtype). */
void orc_backward_tokens(const orc_experts_t* ex, int T, int E, const void* x, int xdt,
                         const void* w_router, int rdt, const double* lam, const int32_t* idx,
                         double scale, const double* dy, const int32_t* tokens, int n_tok,
                         double* dx, double* dweight, double* dlogit, double* y, int nthreads);
void orc_backward_expert_weights(const orc_experts_t* ex, int T, int E, const void* x, int xdt,
                                 const double* lam, const int32_t* idx, double scale,
                                 const double* dy, int e, double* dwg, double* dwu, double* dwd,
                                 int nthreads);
void orc_router_weight_grad(int T, int E, int H, const void* x, int xdt, const double* dlogit,
                            double* dwr);
void orc_logits_any(int T, int H, int E, const void* x, int xdt, const void* w_router, int rdt,
                    double* lam);

#ifdef __cplusplus
}
#endif
#endif
