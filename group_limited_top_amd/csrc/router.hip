// router.hip -- router logits, sigma32 and group-limited top-k selection.
//
// Method: page "InternLumina-U2中256个专家的路由秘密：分组受限Top-K、Expert Bias与
// Fused MoE详解" ([Routing §n] below), §二 steps 1-3 and §三.
#include "device.h"
#include "kernels.h"

#include <math.h>

namespace moe {

// ----------------------------------------------------------------------------
// sigma32: the router sigmoid, specified in include/moe.h.  All operations are
// IEEE fp64 (v_fma_f64, v_rndne_f64, v_div_* correctly rounded division) and
// the final conversion rounds to nearest even, so the value is reproducible
// bit for bit by any IEEE implementation of the same steps.
// ----------------------------------------------------------------------------
__device__ __forceinline__ float sigmoid32(float z) {
  if (!(z == z)) return z;
  const double t = -(double)z;
  if (t > 104.0) return 0.0f;  // below 2^-150: rounds to +0
  if (t < -40.0) return 1.0f;  // exp(t) < 2^-54: 1 + exp(t) rounds to 1
  // Cody-Waite reduction t = n ln2 + r with ln2 = L1 + L2
  const double n = __builtin_rint(t * 0x1.71547652b82fep+0);
  double r = __builtin_fma(-n, 0x1.62e42fefa39efp-1, t);
  r = __builtin_fma(-n, 0x1.abc9e3b39803fp-56, r);
  // exp(r) by the degree-13 Taylor polynomial, coefficients RN(1/i!), Horner
  double p = 0x1.6124613a86d09p-33;          // 1/13!
  p = __builtin_fma(p, r, 0x1.1eed8eff8d898p-29);  // 1/12!
  p = __builtin_fma(p, r, 0x1.ae64567f544e4p-26);  // 1/11!
  p = __builtin_fma(p, r, 0x1.27e4fb7789f5cp-22);  // 1/10!
  p = __builtin_fma(p, r, 0x1.71de3a556c734p-19);  // 1/9!
  p = __builtin_fma(p, r, 0x1.a01a01a01a01ap-16);  // 1/8!
  p = __builtin_fma(p, r, 0x1.a01a01a01a01ap-13);  // 1/7!
  p = __builtin_fma(p, r, 0x1.6c16c16c16c17p-10);  // 1/6!
  p = __builtin_fma(p, r, 0x1.1111111111111p-7);   // 1/5!
  p = __builtin_fma(p, r, 0x1.5555555555555p-5);   // 1/4!
  p = __builtin_fma(p, r, 0x1.5555555555555p-3);   // 1/3!
  p = __builtin_fma(p, r, 0x1.0p-1);               // 1/2!
  p = __builtin_fma(p, r, 1.0);                    // 1/1!
  p = __builtin_fma(p, r, 1.0);                    // 1/0!
  // 2^n is exact: -58 <= n <= 151 here
  const double two_n = __longlong_as_double((long long)((int)n + 1023) << 52);
  const double e = p * two_n;
  const double den = 1.0 + e;
  return (float)(1.0 / den);
}

__global__ void k_sigmoid32(const float* __restrict__ z, float* __restrict__ out, int64_t n) {
  int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (; i < n; i += stride) out[i] = sigmoid32(z[i]);
}

hipError_t launch_sigmoid32(const float* z, float* out, int64_t n, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  int64_t blocks = (n + 255) / 256;
  if (blocks > 65536) blocks = 65536;
  hipLaunchKernelGGL(k_sigmoid32, dim3((unsigned)blocks), dim3(256), 0, s, z, out, n);
  return hipGetLastError();
}

// ----------------------------------------------------------------------------
// Router weight split: w = hi + mid + lo exactly, each part bf16.
// Each step subtracts the nearest bf16 of what is left; the remainder of an
// fp32 after removing its top 8 significant bits, twice, has at most 8
// significant bits, so the three parts represent w exactly.  With bf16 x every
// product x*part is then exact in fp32 and only the accumulation rounds.
// Layout: split[p][e][h], p = 0 (hi), 1 (mid), 2 (lo).
// ----------------------------------------------------------------------------
__global__ void k_split_router(const float* __restrict__ w, uint16_t* __restrict__ split,
                               int64_t n) {
  int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (; i < n; i += stride) {
    const float v = w[i];
    const uint32_t hi = f32_to_bf16_bits(v);
    const float r1 = v - bf16_to_f32((uint16_t)hi);
    const uint32_t mid = f32_to_bf16_bits(r1);
    const float r2 = r1 - bf16_to_f32((uint16_t)mid);
    const uint32_t lo = f32_to_bf16_bits(r2);
    split[i] = (uint16_t)hi;
    split[n + i] = (uint16_t)mid;
    split[2 * n + i] = (uint16_t)lo;
  }
}

hipError_t launch_split_router(const float* w, uint16_t* split, int E, int H, hipStream_t s,
                               const StageTimer* tm) {
  const int64_t n = (int64_t)E * H;
  int64_t blocks = (n + 255) / 256;
  if (blocks > 8192) blocks = 8192;
  stage_begin(tm, kSplit, s);
  hipLaunchKernelGGL(k_split_router, dim3((unsigned)blocks), dim3(256), 0, s, w, split, n);
  stage_end(tm, kSplit, s);
  return hipGetLastError();
}

// ----------------------------------------------------------------------------
// Logits, bf16 activations: logits[t][e] = sum_h x[t][h] * w[e][h] on MFMA with
// w split three ways (hi, mid, lo).  Block = 4 waves; block tile 16 tokens x
// 64 experts, each wave 16 x 16.  [Routing §二 step 1]: linear layer in fp32,
// no bias term.
// ----------------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_logits_bf16(const uint16_t* __restrict__ x,
                                                      const uint16_t* __restrict__ split,
                                                      float* __restrict__ logits, int T, int H,
                                                      int E) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int r = lane & 15, q = lane >> 4;
  const int t0 = blockIdx.x * 16;
  const int e0 = blockIdx.y * 64 + wave * 16;
  if (e0 >= E) return;  // wave-uniform; this kernel has no barrier
  const int ta = min(t0 + r, T - 1);
  const int eb = min(e0 + r, E - 1);
  const size_t EH = (size_t)E * H;
  const uint16_t* xa = x + (size_t)ta * H + q * 8;
  const uint16_t* wb = split + (size_t)eb * H + q * 8;
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  for (int k = 0; k < H; k += 32) {
    const u32x4 a = ld16(xa + k);
    const u32x4 b0 = ld16(wb + k);
    const u32x4 b1 = ld16(wb + EH + k);
    const u32x4 b2 = ld16(wb + 2 * EH + k);
    acc = mfma16x16x32(a, b0, acc);
    acc = mfma16x16x32(a, b1, acc);
    acc = mfma16x16x32(a, b2, acc);
  }
  // C rows are tokens (A), columns experts (B): lane holds C[4q + i][r]
  const int e = e0 + r;
  if (e < E) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int t = t0 + 4 * q + i;
      if (t < T) logits[(size_t)t * E + e] = acc[i];
    }
  }
}

hipError_t launch_logits_bf16(const uint16_t* x, const uint16_t* split, float* logits, int T, int H,
                              int E, hipStream_t s, const StageTimer* tm) {
  dim3 grid((unsigned)((T + 15) / 16), (unsigned)((E + 63) / 64));
  stage_begin(tm, kLogits, s);
  hipLaunchKernelGGL(k_logits_bf16, grid, dim3(256), 0, s, x, split, logits, T, H, E);
  stage_end(tm, kLogits, s);
  return hipGetLastError();
}

// ----------------------------------------------------------------------------
// Logits, fp32 activations (small fp32 layers): one block per token, x row in
// LDS, one thread per expert, fp32 fma in ascending h.
// ----------------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_logits_f32(const float* __restrict__ x,
                                                     const float* __restrict__ w,
                                                     float* __restrict__ logits, int H, int E) {
  extern __shared__ float xs[];
  const int t = blockIdx.x;
  for (int h = threadIdx.x; h < H; h += blockDim.x) xs[h] = x[(size_t)t * H + h];
  __syncthreads();
  for (int e = threadIdx.x; e < E; e += blockDim.x) {
    const float* wr = w + (size_t)e * H;
    float acc = 0.0f;
    for (int h = 0; h < H; h += 4) {
      const float4 v = *reinterpret_cast<const float4*>(wr + h);
      acc = __builtin_fmaf(xs[h], v.x, acc);
      acc = __builtin_fmaf(xs[h + 1], v.y, acc);
      acc = __builtin_fmaf(xs[h + 2], v.z, acc);
      acc = __builtin_fmaf(xs[h + 3], v.w, acc);
    }
    logits[(size_t)t * E + e] = acc;
  }
}

hipError_t launch_logits_f32(const float* x, const float* w, float* logits, int T, int H, int E,
                             hipStream_t s, const StageTimer* tm) {
  stage_begin(tm, kLogits, s);
  hipLaunchKernelGGL(k_logits_f32, dim3((unsigned)T), dim3(256), (size_t)H * sizeof(float), s, x, w,
                     logits, H, E);
  stage_end(tm, kLogits, s);
  return hipGetLastError();
}

// ----------------------------------------------------------------------------
// Selection.  One 64-lane block per token.
//   [Routing §二 step 1]  s = sigma32(logit) per expert
//   [Routing §三]         sb = s + bias (selection only)
//   [Routing §二 step 2]  groups = contiguous ranges of E/n_group experts; group
//                         score = sum of its two largest sb; keep topk_group
//                         groups (ties: lower group); others masked to -inf;
//                         top_k of the rest by (sb desc, expert asc)
//   [Routing §二 step 3]  w_j = RN(RN(s_j / RN(S + 1e-20)) * scale), S the fp32
//                         sum of the chosen unbiased scores in choice order
// ----------------------------------------------------------------------------
constexpr int kMaxE = 512;
constexpr int kMaxTopK = 16;

__global__ __launch_bounds__(64) void k_select(const float* __restrict__ logits,
                                                const float* __restrict__ bias,
                                                int32_t* __restrict__ idx, float* __restrict__ wout,
                                                uint32_t* __restrict__ status, int E, int n_group,
                                                int topk_group, int K, float scale, int record) {
  __shared__ float s_s[kMaxE];
  __shared__ float s_sb[kMaxE];
  __shared__ float s_gs[64];
  __shared__ int s_keep[64];
  __shared__ int s_sel[kMaxTopK];
  const int t = blockIdx.x;
  const int lane = threadIdx.x;
  const float* lg = logits + (size_t)t * E;

  int bad = 0;
  for (int e = lane; e < E; e += 64) {
    const float z = lg[e];
    const float s = sigmoid32(z);
    const float sb = s + (bias ? bias[e] : 0.0f);
    bad |= !(__builtin_isfinite(z) && __builtin_isfinite(sb));
    s_s[e] = s;
    s_sb[e] = sb;
  }
  if (__any(bad)) {  // block-uniform: the block is one wave
    if (lane < K) {
      idx[(size_t)t * K + lane] = lane;
      wout[(size_t)t * K + lane] = 0.0f;
    }
    if (lane == 0 && record) atomicOr(status, 1u);
    return;
  }
  __syncthreads();

  const int gsize = E / n_group;
  if (lane < n_group) {
    float m1 = -INFINITY, m2 = -INFINITY;
    const float* g = s_sb + lane * gsize;
    for (int i = 0; i < gsize; ++i) {
      const float v = g[i];
      if (v > m1) {
        m2 = m1;
        m1 = v;
      } else if (v > m2) {
        m2 = v;
      }
    }
    s_gs[lane] = m1 + m2;
  }
  __syncthreads();
  if (lane < n_group) {
    const float mine = s_gs[lane];
    int rank = 0;
    for (int o = 0; o < n_group; ++o) {
      const float v = s_gs[o];
      rank += (v > mine) || (v == mine && o < lane);
    }
    s_keep[lane] = rank < topk_group;
  }
  __syncthreads();

  // each lane holds experts lane + 64*m, masked to -inf outside kept groups
  float v[kMaxE / 64];
#pragma unroll
  for (int m = 0; m < kMaxE / 64; ++m) {
    const int e = lane + 64 * m;
    v[m] = (e < E) ? (s_keep[e / gsize] ? s_sb[e] : -INFINITY) : -INFINITY;
  }
  uint32_t taken = 0;
  float S = 0.0f;
  for (int j = 0; j < K; ++j) {
    float bv = -INFINITY;
    int be = 0x7fffffff;
    int have = 0;
#pragma unroll
    for (int m = 0; m < kMaxE / 64; ++m) {
      const int e = lane + 64 * m;
      if (e < E && !((taken >> m) & 1u) && (!have || v[m] > bv)) {
        bv = v[m];
        be = e;
        have = 1;
      }
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
      const float ov = __shfl_xor(bv, off);
      const int oe = __shfl_xor(be, off);
      const int oh = __shfl_xor(have, off);
      const bool better = oh && (!have || ov > bv || (ov == bv && oe < be));
      if (better) {
        bv = ov;
        be = oe;
        have = oh;
      }
    }
    if ((be & 63) == lane) taken |= 1u << (be >> 6);
    if (lane == 0) {
      s_sel[j] = be;
      S = (j == 0) ? s_s[be] : S + s_s[be];
    }
  }
  if (lane == 0) {
    const float d = S + 1e-20f;
    for (int j = 0; j < K; ++j) {
      const int e = s_sel[j];
      const float qv = s_s[e] / d;
      idx[(size_t)t * K + j] = e;
      wout[(size_t)t * K + j] = qv * scale;
    }
  }
}

hipError_t launch_select(const float* logits, const float* bias, int32_t* idx, float* w,
                         uint32_t* status, int T, int E, int n_group, int topk_group, int K,
                         float scale, bool record_nonfinite, hipStream_t s,
                         const StageTimer* tm) {
  stage_begin(tm, kSelect, s);
  hipLaunchKernelGGL(k_select, dim3((unsigned)T), dim3(64), 0, s, logits, bias, idx, w, status, E,
                     n_group, topk_group, K, scale, record_nonfinite ? 1 : 0);
  stage_end(tm, kSelect, s);
  return hipGetLastError();
}

}  // namespace moe
